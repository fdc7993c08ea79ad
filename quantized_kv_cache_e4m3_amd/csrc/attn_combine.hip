// Combine step of split-T attention: merge the (m, l, acc) partials of the
// row chunks of every query row, then (TQ4) rotate the merged context back
// once per head.  [colibri #399] "Commits" item 2 (split-T kernels with a
// merge) and "Ready for review" comment (unrotate the accumulated context once).
//
//   M = max_j m_j,  out = sum_j e^(m_j - M) acc_j / sum_j e^(m_j - M) l_j,
//   lse = M + ln(sum_j e^(m_j - M) l_j)
//
// One workgroup per (query row, 64-dim slice) with one wave per 64 chunks (at
// most 16 waves).  Wave w takes its share of the chunks, in rounds of 64: lane
// j holds the (m, l) of chunk base + j, each chunk's weight reaches the other
// lanes by readlane, and lane i sums the chunks' values of dim slice + i in
// chunk order.  A round's (m, l) load is issued before its 32 value loads,
// with no branch (loads return in issue order), so the weights are computed
// while the values are in flight; rounds and then the waves merge like an
// online softmax.  (32 chunks per round: the round's 33 loads fit the 63 a
// wave can have in flight, so they wait once; with 64 the compiler split the
// value loads around a wait, and the 64-chunk decode now takes two waves per
// slice and their merge: KV8 decode -0.4 to -0.6 us in same-box A/B.)
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kSlice = 64;
constexpr int kMaxSplit = 4096;
constexpr int kRound = 32;
constexpr int kMaxWaves = 16;

__device__ __forceinline__ double xor_lane_d(double v, int m) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __shfl_xor((int)(uint32_t)b, m), hi = __shfl_xor((int)(uint32_t)(b >> 32), m);
    return __builtin_bit_cast(double, (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32));
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += xor_lane_d(v, m);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
    v += xor_lane<32>(v);
    v += xor_lane<16>(v);
    v += xor_lane<8>(v);
    v += xor_lane<4>(v);
    v += xor_lane<2>(v);
    v += xor_lane<1>(v);
    return v;
}

__global__ __launch_bounds__(64 * kMaxWaves) void k_combine(const float* __restrict__ part_acc,
                                                 const float* __restrict__ part_ml, int n_split,
                                                 int64_t n_qrows, int d, bool log2_domain,
                                                 float* __restrict__ out, float* __restrict__ lse) {
    __shared__ float m_s[kMaxWaves];
    __shared__ double l_s[kMaxWaves];
    __shared__ double s_s[kMaxWaves][kSlice];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int c = blockIdx.y * kSlice + lane;
    const bool act = c < d;
    const float* src = part_acc + r * d + (act ? c : 0);
    const int64_t stride = n_qrows * d;
    const int nw = blockDim.x >> 6;
    const int per = (n_split + nw - 1) / nw;
    const int j0 = wv * per, j1 = (j0 + per < n_split) ? j0 + per : n_split;
    auto ex = [&](float x) { return log2_domain ? exp2f(x) : expf(x); };

    // the weighted sums in f64: with hundreds of chunks their f32 rounding
    // would be a visible part of the error budget
    float M = -INFINITY;
    double s = 0.0, lpart = 0.0;
    for (int base = j0; base < j1; base += kRound) {
        const int last = j1 - 1;
        // lane j < kRound: chunk base + j's (m, l), loaded first and with no
        // branch (a lane past the round reads chunk base and drops it), so the
        // round's loads are in flight together and wait once
        const bool own = lane < kRound && base + lane < j1;
        const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((int64_t)(own ? base + lane : base) * n_qrows + r) * 2);
        const float m = own ? ml.x : -INFINITY;
        const float l = own ? ml.y : 0.0f;
        // a chunk past the wave's range reads its last chunk (finite) and gets weight 0
        float v[kRound];
#pragma unroll
        for (int u = 0; u < kRound; ++u) v[u] = src[(int64_t)(base + u < j1 ? base + u : last) * stride];
        const float Mn = fmaxf(M, wave_max(m));
        const float a_old = (M == -INFINITY) ? 0.0f : ex(M - Mn);
        const float w = (m == -INFINITY) ? 0.0f : ex(m - Mn);
        s *= a_old;
        lpart = lpart * a_old + (double)w * l;
        M = Mn;
#pragma unroll
        for (int u = 0; u < kRound; ++u) {
            const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
            s = fma((double)wu, (double)v[u], s);
        }
    }
    const double L = wave_sum_d(lpart);
    if (lane == 0) {
        m_s[wv] = M;
        l_s[wv] = L;
    }
    s_s[wv][lane] = s;
    __syncthreads();
    if (wv != 0) return;
    float Mt = -INFINITY;
    for (int k = 0; k < nw; ++k) Mt = fmaxf(Mt, m_s[k]);
    double st = 0.0, Lt = 0.0;
    for (int k = 0; k < nw; ++k) {
        const double f = (m_s[k] == -INFINITY) ? 0.0 : (double)ex(m_s[k] - Mt);
        st += f * s_s[k][lane];
        Lt += f * l_s[k];
    }
    if (act) out[r * d + c] = Lt > 0.0 ? (float)(st / Lt) : 0.0f;      // no row at all: 0 (lse -inf)
    if (lse != nullptr && blockIdx.y == 0 && lane == 0)
        lse[r] = log2_domain ? (Mt + (float)log2(Lt)) * 0.69314718055994531f : Mt + (float)log(Lt);
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

// The same at d = 512, one wave per row in registers: lane l holds dims
// 8l .. 8l+7, the strides 1 .. 4 stay inside the lane and 8 .. 256 are lane
// swaps (the same butterflies in the same order as above).
__global__ __launch_bounds__(64) void k_unrotate512(float* __restrict__ out, uint64_t seed) {
    constexpr int DD = 512;
    const int64_t r = blockIdx.x;
    const int lane = threadIdx.x;
    float* row = out + r * DD + 8 * lane;
    const float4 u0 = *reinterpret_cast<const float4*>(row);
    const float4 u1 = *reinterpret_cast<const float4*>(row + 4);
    float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & h) continue;
            const float a = v[i], b = v[i + h];
            v[i] = a + b;
            v[i + h] = a - b;
        }
    }
    auto stage = [&](auto xl, int m) {
        const bool upper = (lane >> m) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float o = xl(v[e]);
            v[e] = upper ? (o - v[e]) : (v[e] + o);
        }
    };
    stage([](float x) { return xor_lane<1>(x); }, 0);
    stage([](float x) { return xor_lane<2>(x); }, 1);
    stage([](float x) { return xor_lane<4>(x); }, 2);
    stage([](float x) { return xor_lane<8>(x); }, 3);
    stage([](float x) { return xor_lane<16>(x); }, 4);
    stage([](float x) { return xor_lane<32>(x); }, 5);
    const uint64_t w = splitmix64_at(seed, (uint64_t)(lane >> 3));
    const int sh = 8 * (lane & 7);
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if ((w >> (sh + e)) & 1ull) v[e] = -v[e];
    *reinterpret_cast<float4*>(row) = float4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<float4*>(row + 4) = float4{v[4], v[5], v[6], v[7]};
}

// TQ4 at d = 512: the merge and the inverse rotation in one workgroup per
// query row.  Wave w merges dims 64w .. 64w + 63 over all chunks (every wave
// derives the same M and L from the chunks' (m, l)); lane j of a round holds
// chunk base + j's (m, l), issued ahead of the round's 64 chunk values.  The
// merged row then goes through the FWHT (stages below 64 by lane swaps inside
// each wave, the three larger ones through LDS) and the sign flips.
__global__ __launch_bounds__(512) void k_combine_unrotate512(const float* __restrict__ part_acc,
                                                            const float* __restrict__ part_ml,
                                                            int n_split, int64_t n_qrows,
                                                            bool log2_domain, uint64_t seed,
                                                            float* __restrict__ out,
                                                            float* __restrict__ lse) {
    constexpr int DD = 512;
    __shared__ float o_s[2 * DD];
    const int64_t r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int c = tid;                                  // wave w: dims 64w + lane
    const float* src = part_acc + r * DD + c;
    const int64_t stride = n_qrows * DD;
    const int last = n_split - 1;
    auto ex = [&](float x) { return log2_domain ? exp2f(x) : expf(x); };

    float M = -INFINITY, s = 0.0f, lpart = 0.0f;
    for (int base = 0; base < n_split; base += kSlice) {
        const int jm = base + lane;
        const float2 mlv = *reinterpret_cast<const float2*>(part_ml + ((int64_t)(jm < n_split ? jm : last) * n_qrows + r) * 2);
        const float m = jm < n_split ? mlv.x : -INFINITY;
        const float l = jm < n_split ? mlv.y : 0.0f;
        // a chunk past n_split reads chunk n_split - 1 (finite) and gets weight 0
        float v[kSlice];
#pragma unroll
        for (int u = 0; u < kSlice; ++u) v[u] = src[(int64_t)(base + u < n_split ? base + u : last) * stride];
        const float Mn = fmaxf(M, wave_max(m));
        const float a_old = (M == -INFINITY) ? 0.0f : ex(M - Mn);
        const float w = (m == -INFINITY) ? 0.0f : ex(m - Mn);
        s *= a_old;
        lpart = lpart * a_old + w * l;
        M = Mn;
#pragma unroll
        for (int u = 0; u < kSlice; ++u) {
            const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), u));
            s = fmaf(wu, v[u], s);
        }
    }
    const float L = wave_sum(lpart);
    float v = L > 0.0f ? s / L : 0.0f;                 // no row at all: 0 (lse -inf)
    if (lse != nullptr && tid == 0)
        lse[r] = log2_domain ? (M + log2f(L)) * 0.69314718055994531f : M + logf(L);
    // out <- D (H out): butterflies h = 1 .. 256 (the lower element of a pair
    // keeps a + b, the upper one a - b), then the encoder's signs.  Stages
    // h < 64 pair lanes of one wave; h = 64, 128, 256 pair waves, through a
    // double-buffered LDS row (one barrier per stage).
    auto bfly = [&](float o, bool upper) { return upper ? (o - v) : (v + o); };
    v = bfly(xor_lane<1>(v), (c & 1) != 0);
    v = bfly(xor_lane<2>(v), (c & 2) != 0);
    v = bfly(xor_lane<4>(v), (c & 4) != 0);
    v = bfly(xor_lane<8>(v), (c & 8) != 0);
    v = bfly(xor_lane<16>(v), (c & 16) != 0);
    v = bfly(xor_lane<32>(v), (c & 32) != 0);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int h = 64 << k;
        float* buf = o_s + (k & 1) * DD;
        buf[c] = v;
        __syncthreads();
        v = bfly(buf[c ^ h], (c & h) != 0);
    }
    const uint64_t wd = splitmix64_at(seed, (uint64_t)(c >> 6));
    out[r * DD + c] = ((wd >> (c & 63)) & 1ull) ? -v : v;
}

}  // namespace

hipError_t launch_combine(int32_t fmt, const float* part_acc, const float* part_ml, int n_split,
                          int64_t n_qrows, int d, uint64_t seed, bool log2_domain, float* out,
                          float* lse, hipStream_t s) {
    if (n_split > kMaxSplit) return hipErrorInvalidValue;
    // (the fused merge-and-unrotate takes one workgroup per query row, which
    // keeps up with up to 64 chunks; more chunks are merged by the sliced
    // kernel and unrotated after it)
    if (fmt == KVQ_TQ4 && d == 512 && n_split <= 64) {
        k_combine_unrotate512<<<(unsigned)n_qrows, 512, 0, s>>>(part_acc, part_ml, n_split, n_qrows,
                                                                log2_domain, seed, out, lse);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)n_qrows, (unsigned)((d + kSlice - 1) / kSlice));
    int waves = (n_split + kRound - 1) / kRound;
    waves = waves < 1 ? 1 : (waves > kMaxWaves ? kMaxWaves : waves);
    k_combine<<<grid, 64 * waves, 0, s>>>(part_acc, part_ml, n_split, n_qrows, d, log2_domain, out, lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fmt != KVQ_TQ4) return e;
    return launch_unrotate(out, n_qrows, d, seed, s);
}

hipError_t launch_unrotate(float* out, int64_t n_qrows, int d, uint64_t seed, hipStream_t s) {
    if (d == 512 && reinterpret_cast<uintptr_t>(out) % 16 == 0)
        k_unrotate512<<<(unsigned)n_qrows, 64, 0, s>>>(out, seed);
    else
        k_unrotate<<<(unsigned)n_qrows, 256, sizeof(float) * d, s>>>(out, d, seed);
    return hipGetLastError();
}

}  // namespace kvq
