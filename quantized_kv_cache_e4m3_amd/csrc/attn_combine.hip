// Combine step of split-T attention: merge the (m, l, acc) partials of the
// row chunks of every query row, then (TQ4) rotate the merged context back
// once per head.  [colibri #399] "Commits" item 2 (split-T kernels with a
// merge) and "Ready for review" comment (unrotate the accumulated context once).
//
//   M = max_j m_j,  out = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j,
//   lse = M + ln(sum_j e^(m_j - M) l_j)
//
// One workgroup per (query row, 64-dim slice): 4 groups of 64 threads each
// sum a quarter of the chunks for the slice's 64 dims, then add in LDS.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kSlice = 64;
constexpr int kMaxSplit = 4096;

__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ part_acc,
                                                 const float* __restrict__ part_ml, int n_split,
                                                 int64_t n_qrows, int d, bool log2_domain,
                                                 float* __restrict__ out, float* __restrict__ lse) {
    __shared__ float w_s[kMaxSplit];
    __shared__ float red_s[2][4];
    __shared__ float sum_s[4][kSlice];
    const int64_t r = blockIdx.x;
    const int c0 = blockIdx.y * kSlice;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

    float mx = -INFINITY;
    for (int j = tid; j < n_split; j += 256) mx = fmaxf(mx, part_ml[((int64_t)j * n_qrows + r) * 2]);
    mx = wave_max(mx);
    if (lane == 0) red_s[0][wv] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red_s[0][0], red_s[0][1]), fmaxf(red_s[0][2], red_s[0][3]));
    float lsum = 0.0f;
    for (int j = tid; j < n_split; j += 256) {
        const float* ml = part_ml + ((int64_t)j * n_qrows + r) * 2;
        const float w = (ml[0] == -INFINITY) ? 0.0f
                        : (log2_domain ? exp2f(ml[0] - M) : expf(ml[0] - M));
        w_s[j] = w;
        lsum += w * ml[1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lsum += __shfl_xor(lsum, o);
    if (lane == 0) red_s[1][wv] = lsum;
    __syncthreads();
    const float L = (red_s[1][0] + red_s[1][1]) + (red_s[1][2] + red_s[1][3]);

    // each group of 64 threads sums every 4th chunk for the slice's 64 dims,
    // 8 independent loads in flight per thread
    const int grp = wv, c = c0 + lane;
    float s = 0.0f;
    if (c < d) {
        const float* src = part_acc + r * d + c;
        const int64_t stride = n_qrows * d;
        int j = grp;
        for (; j + 28 < n_split; j += 32) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(j + 4 * u) * stride];
#pragma unroll
            for (int u = 0; u < 8; ++u) s = fmaf(w_s[j + 4 * u], v[u], s);
        }
        for (; j < n_split; j += 4) s = fmaf(w_s[j], src[(int64_t)j * stride], s);
    }
    sum_s[grp][tid & 63] = s;
    __syncthreads();
    if (grp == 0 && c < d) {
        const float t = (sum_s[0][tid] + sum_s[1][tid]) + (sum_s[2][tid] + sum_s[3][tid]);
        out[r * d + c] = t / L;
    }
    if (lse != nullptr && blockIdx.y == 0 && tid == 0)
        lse[r] = log2_domain ? (M + log2f(L)) * 0.69314718055994531f : M + logf(L);
}

// out_h <- D (H out_h): the inverse of the encoder's rotation for the merged
// rotated-domain context (the 1/d is already in the row weights).
__global__ __launch_bounds__(256) void k_unrotate(float* __restrict__ out, int d, uint64_t seed) {
    extern __shared__ float o_s[];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x;
    for (int c = tid; c < d; c += 256) o_s[c] = out[r * d + c];
    __syncthreads();
    for (int h = 1; h < d; h <<= 1) {
        for (int p = tid; p < d / 2; p += 256) {
            const int i = (p / h) * 2 * h + (p % h);
            const float x0 = o_s[i], x1 = o_s[i + h];
            o_s[i] = x0 + x1;
            o_s[i + h] = x0 - x1;
        }
        __syncthreads();
    }
    for (int c = tid; c < d; c += 256) {
        const uint64_t w = splitmix64_at(seed, (uint64_t)(c >> 6));
        const float v = o_s[c];
        out[r * d + c] = ((w >> (c & 63)) & 1ull) ? -v : v;
    }
}

}  // namespace

hipError_t launch_combine(int32_t fmt, const float* part_acc, const float* part_ml, int n_split,
                          int64_t n_qrows, int d, uint64_t seed, bool log2_domain, float* out,
                          float* lse, hipStream_t s) {
    if (n_split > kMaxSplit) return hipErrorInvalidValue;
    const dim3 grid((unsigned)n_qrows, (unsigned)((d + kSlice - 1) / kSlice));
    k_combine<<<grid, 256, 0, s>>>(part_acc, part_ml, n_split, n_qrows, d, log2_domain, out, lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fmt != KVQ_TQ4) return e;
    return launch_unrotate(out, n_qrows, d, seed, s);
}

hipError_t launch_unrotate(float* out, int64_t n_qrows, int d, uint64_t seed, hipStream_t s) {
    k_unrotate<<<(unsigned)n_qrows, 256, sizeof(float) * d, s>>>(out, d, seed);
    return hipGetLastError();
}

}  // namespace kvq
