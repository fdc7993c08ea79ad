// Encoders (the producer side) for gfx950: KV8, rotated-int4 (TQ4) and q2k.
//
// Every stored byte is decided by f32 arithmetic whose order is fixed here
// (the library is built with -ffp-contract=off, so no multiply-add is fused
// and every add / multiply / divide / sqrt is one IEEE rounding; the one
// explicit fma, in the d = 512 TQ4 encoder, has an exact product).
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kRowsPerBlock = 4;   // one 64-lane wave per row, 4 waves per workgroup
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// KV8: fp8 e4m3 codes + f32 scale = amax/448 per row.
// [colibri #399] "Summary" / "Commits" item 1; [colibri #553] "What's in it".
// ---------------------------------------------------------------------------

// (the e4m3 conversion of a quotient, sat448 and e4m3x4, is shared with the
// decode that encodes its appended row itself)

// d % 8 == 0 and d <= 512 * J: lane L owns 8-float chunks L, L+64, ...
template <int J>
__global__ __launch_bounds__(256) void k_encode_fp8_vec(const float* __restrict__ x, int64_t n_rows,
                                                        int d, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const float* xr = x + row * (int64_t)d;
    const int nchunk = d >> 3;
    float v[J][8];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        if (c < nchunk) {
            const float4 a = *reinterpret_cast<const float4*>(xr + 8 * c);
            const float4 b = *reinterpret_cast<const float4*>(xr + 8 * c + 4);
            v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
            v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[j][e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[j][e]));
    }
    amax = wave_max(amax);
    const float s = amax / 448.0f;
    const bool live = s > 0.0f;
    if (lane == 0) scales[row] = live ? s : 0.0f;
    uint8_t* cr = codes + row * (int64_t)d;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = lane + 64 * j;
        if (c < nchunk) {
            uint32_t w0 = 0, w1 = 0;
            if (live) {
                w0 = e4m3x4(v[j][0] / s, v[j][1] / s, v[j][2] / s, v[j][3] / s);
                w1 = e4m3x4(v[j][4] / s, v[j][5] / s, v[j][6] / s, v[j][7] / s);
            }
            *reinterpret_cast<uint2*>(cr + 8 * c) = make_uint2(w0, w1);
        }
    }
}

// Any d: one wave per row, lane-strided elements, byte stores.
__global__ __launch_bounds__(256) void k_encode_fp8_any(const float* __restrict__ x, int64_t n_rows,
                                                        int d, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const float* xr = x + row * (int64_t)d;
    float amax = 0.0f;
    for (int i = lane; i < d; i += 64) amax = fmaxf(amax, fabsf(xr[i]));
    amax = wave_max(amax);
    const float s = amax / 448.0f;
    const bool live = s > 0.0f;
    if (lane == 0) scales[row] = live ? s : 0.0f;
    uint8_t* cr = codes + row * (int64_t)d;
    for (int i = lane; i < d; i += 64)
        cr[i] = live ? (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(sat448(xr[i] / s), 0.0f, 0, false) & 0xFF)
                     : (uint8_t)0;
}

// ---------------------------------------------------------------------------
// TQ4: radius, randomized Walsh-Hadamard rotation, 16-level codebook, nibbles.
// [colibri #399] "Why rotated-int4 for the 4-bit tier"; [colibri #553].
// Lane L owns the E contiguous elements E*L .. E*L+E-1 (d >= 64: E = d/64;
// d < 64: E = 1 and lanes L < d).  Transform stages with h < E stay in
// registers, the others pair lanes L and L ^ (h/E).
// ---------------------------------------------------------------------------
template <int E>
__global__ __launch_bounds__(256) void k_encode_tq4(const float* __restrict__ x, int64_t n_rows,
                                                    int d, uint64_t seed, Codebook16 cb,
                                                    uint8_t* __restrict__ packed,
                                                    float* __restrict__ radius) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
    if (row >= n_rows) return;
    const int nl = d / E;                   // active lanes
    const bool act = lane < nl;
    const float* xr = x + row * (int64_t)d + (int64_t)E * lane;
    float v[E];
    if constexpr (E >= 4) {
#pragma unroll
        for (int j = 0; j < E; j += 4) {
            const float4 a = *reinterpret_cast<const float4*>(xr + j);
            v[j] = a.x; v[j + 1] = a.y; v[j + 2] = a.z; v[j + 3] = a.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < E; ++j) v[j] = act ? xr[j] : 0.0f;
    }

    // radius: p_i = x_i^2; for h = d/2 .. 1: p_i += p_{i+h} (i < h); r = sqrt(p_0)
    float p[E];
#pragma unroll
    for (int j = 0; j < E; ++j) p[j] = v[j] * v[j];
    for (int h = d >> 1; h >= E; h >>= 1) {
        const int m = h / E;
#pragma unroll
        for (int j = 0; j < E; ++j) p[j] = p[j] + __shfl_xor(p[j], m);
    }
#pragma unroll
    for (int h = E >> 1; h >= 1; h >>= 1) {
#pragma unroll
        for (int j = 0; j < h; ++j) p[j] = p[j] + p[j + h];
    }
    const float ss = __shfl(p[0], 0);
    const float r = sqrtf(ss);

    // sign diagonal: element i flips when bit i%64 of SplitMix64 output i/64 is set
    {
        const int i0 = E * lane;
        const uint64_t w = splitmix64_at(seed, (uint64_t)(i0 >> 6));
        const int b0 = i0 & 63;
#pragma unroll
        for (int j = 0; j < E; ++j)
            if ((w >> (b0 + j)) & 1ull) v[j] = -v[j];
    }
    // unnormalised Walsh-Hadamard: stages h = 1, 2, ..., d/2
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
            if ((j & h) == 0) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    for (int h = (E > 1 ? E : 1); h < d; h <<= 1) {
        const int m = h / E;
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            const float o = __shfl_xor(v[j], m);
            v[j] = upper ? (o - v[j]) : (v[j] + o);
        }
    }

    // level = number of thresholds fl32(tau_k * r) strictly below y
    float t[15];
#pragma unroll
    for (int k = 0; k < 15; ++k) t[k] = cb.thr[k] * r;
    const bool live = r > 0.0f;
    uint32_t idx[E];
#pragma unroll
    for (int j = 0; j < E; ++j) {
        uint32_t c = 0;
#pragma unroll
        for (int k = 0; k < 15; ++k) c += (v[j] > t[k]) ? 1u : 0u;
        idx[j] = live ? c : 0u;
    }
    if (lane == 0) radius[row] = live ? r : 0.0f;

    uint8_t* pr = packed + row * (int64_t)(d >> 1);
    if constexpr (E == 1) {
        const uint32_t hi = (uint32_t)__shfl_down((int)idx[0], 1);
        if (act && (lane & 1) == 0) pr[lane >> 1] = (uint8_t)(idx[0] | (hi << 4));
    } else if constexpr (E == 2) {
        pr[lane] = (uint8_t)(idx[0] | (idx[1] << 4));
    } else if constexpr (E == 4) {
        const uint32_t w = idx[0] | (idx[1] << 4) | (idx[2] << 8) | (idx[3] << 12);
        *reinterpret_cast<uint16_t*>(pr + 2 * lane) = (uint16_t)w;
    } else {
#pragma unroll
        for (int q = 0; q < E / 8; ++q) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= idx[8 * q + i] << (4 * i);
            *reinterpret_cast<uint32_t*>(pr + (E / 2) * lane + 4 * q) = w;
        }
    }
}

// TQ4 at d = 512 with 8 lanes per row (8 rows per wave).  Lane l holds the
// 64-element block b(l) = l ^ (l & 4 ? 3 : 0) of its row, so the three stages
// that pair elements 64, 128 and 256 apart pair lane l with lane l ^ 1,
// l ^ 2 (quad permutes) and 7 - l (half-row mirror): one DPP move per value.
// The stages 1 .. 32 stay in registers.  The arithmetic and its order are
// those of k_encode_tq4 (radius tree h = 256 .. 1, FWHT stages h = 1 .. 256,
// butterflies (a + b, a - b)), so the bytes are the same; every lane of a row
// ends the radius tree with the row's sum.  The level count is a 4-step
// binary search over the 15 scaled thresholds, which gives #{k : y > T_k}
// because T_k = fl(thr_k * r) is non-decreasing in k for finite r >= 0; a row
// whose radius overflowed (r = inf, T_7 = 0 * inf = NaN) counts linearly.
constexpr int kTq4RowsPerBlock512 = 32;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm(1, 0, 3, 2)
constexpr int kDppXor2 = 0x4E;          // quad_perm(2, 3, 0, 1)
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i inside each group of 8

__global__ __launch_bounds__(256) void k_encode_tq4_512(const float* __restrict__ x, int64_t n_rows,
                                                        uint64_t seed, Codebook16 cb,
                                                        uint8_t* __restrict__ packed,
                                                        float* __restrict__ radius, bool wide_store) {
    constexpr int D = 512, B = 64;
    const int l = threadIdx.x & 7;
    const int64_t row = (int64_t)blockIdx.x * kTq4RowsPerBlock512 + (threadIdx.x >> 3);
    if (row >= n_rows) return;              // whole 8-lane groups: the DPP moves stay inside a row
    const int blk = l ^ ((l & 4) ? 3 : 0);
    const float* xr = x + row * D + B * blk;
    float v[B];
#pragma unroll
    for (int j = 0; j < B; j += 4) {
        const float4 a = *reinterpret_cast<const float4*>(xr + j);
        v[j] = a.x; v[j + 1] = a.y; v[j + 2] = a.z; v[j + 3] = a.w;
    }

    // radius: p_i = x_i^2, then p_i += p_{i+h} for h = 256, 128, 64 (across
    // lanes), 32 .. 1 (in registers); r = sqrt(p_0)
    float r;
    {
        float p[B];
#pragma unroll
        for (int j = 0; j < B; ++j) p[j] = v[j] * v[j];
#pragma unroll
        for (int j = 0; j < B; ++j) p[j] = p[j] + dpp_f<kDppHalfMirror>(p[j]);
#pragma unroll
        for (int j = 0; j < B; ++j) p[j] = p[j] + dpp_f<kDppXor2>(p[j]);
#pragma unroll
        for (int j = 0; j < B; ++j) p[j] = p[j] + dpp_f<kDppXor1>(p[j]);
#pragma unroll
        for (int h = B / 2; h >= 1; h >>= 1)
#pragma unroll
            for (int j = 0; j < h; ++j) p[j] = p[j] + p[j + h];
        r = sqrtf(p[0]);
    }

    // sign diagonal: element 64 blk + j flips when bit j of SplitMix64 output blk is set
    {
        const uint64_t w = splitmix64_at(seed, (uint64_t)blk);
#pragma unroll
        for (int j = 0; j < B; ++j)
            if ((w >> j) & 1ull) v[j] = -v[j];
    }
    // unnormalised Walsh-Hadamard, stages h = 1 .. 32 in registers
#pragma unroll
    for (int h = 1; h < B; h <<= 1) {
#pragma unroll
        for (int j = 0; j < B; ++j) {
            if ((j & h) == 0) {
                const float a = v[j], b = v[j + h];
                v[j] = a + b;
                v[j + h] = a - b;
            }
        }
    }
    // stages 64, 128, 256 across lanes: the lower block of a pair keeps
    // v + o, the upper one o - v (o: the partner's value), as fma(v, +-1, o)
    // with an exact product
    {
        const float s64 = (blk & 1) ? -1.0f : 1.0f;
        const float s128 = (blk & 2) ? -1.0f : 1.0f;
        const float s256 = (blk & 4) ? -1.0f : 1.0f;
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = __builtin_fmaf(v[j], s64, dpp_f<kDppXor1>(v[j]));
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = __builtin_fmaf(v[j], s128, dpp_f<kDppXor2>(v[j]));
#pragma unroll
        for (int j = 0; j < B; ++j) v[j] = __builtin_fmaf(v[j], s256, dpp_f<kDppHalfMirror>(v[j]));
    }

    // level = number of thresholds fl32(thr_k * r) strictly below y
    float t[15];
#pragma unroll
    for (int k = 0; k < 15; ++k) t[k] = cb.thr[k] * r;
    const bool live = r > 0.0f;
    const bool ordered = r < INFINITY;
    uint32_t word[B / 8];
#pragma unroll
    for (int q = 0; q < B / 8; ++q) {
        uint32_t wq = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float y = v[8 * q + i];
            uint32_t c;
            if (ordered) {
                const bool m1 = y > t[7];
                const bool m2 = y > (m1 ? t[11] : t[3]);
                const bool m3 = y > (m1 ? (m2 ? t[13] : t[9]) : (m2 ? t[5] : t[1]));
                const float a0 = m3 ? t[2] : t[0], a1 = m3 ? t[6] : t[4];
                const float a2 = m3 ? t[10] : t[8], a3 = m3 ? t[14] : t[12];
                const float b0 = m2 ? a1 : a0, b1 = m2 ? a3 : a2;
                const bool m4 = y > (m1 ? b1 : b0);
                c = (m1 ? 8u : 0u) + (m2 ? 4u : 0u) + (m3 ? 2u : 0u) + (m4 ? 1u : 0u);
            } else {
                c = 0;
#pragma unroll
                for (int k = 0; k < 15; ++k) c += (y > t[k]) ? 1u : 0u;
            }
            wq |= (live ? c : 0u) << (4 * i);
        }
        word[q] = wq;
    }
    if (l == 0) radius[row] = live ? r : 0.0f;
    uint8_t* pr = packed + row * (D / 2) + (B / 2) * blk;
    if (wide_store) {
        *reinterpret_cast<u32x4*>(pr) = u32x4{word[0], word[1], word[2], word[3]};
        *reinterpret_cast<u32x4*>(pr + 16) = u32x4{word[4], word[5], word[6], word[7]};
    } else {
#pragma unroll
        for (int q = 0; q < B / 8; ++q) *reinterpret_cast<uint32_t*>(pr + 4 * q) = word[q];
    }
}

// ---------------------------------------------------------------------------
// q2k.  [Strata #2318] "Summary" items 1-3, "Why per-channel K and per-token V".
// ---------------------------------------------------------------------------

// K: one thread per (group, head, channel); the 32 cells of the group are
// summed in cell order, codes use the un-gained RMS, the stored scale is
// f16(gain * RMS).
__device__ __forceinline__ void encode_q2k_k_one(int64_t gid, const float* __restrict__ k, int n_kv, int d,
                                                 float gain, const Codebook4& cb,
                                                 uint8_t* __restrict__ k_codes,
                                                 uint16_t* __restrict__ k_scale) {
    // gid = (g, h, c)
    const int c = (int)(gid % d);
    const int64_t gh = gid / d;
    const int h = (int)(gh % n_kv);
    const int64_t g = gh / n_kv;
    const int64_t stride = (int64_t)n_kv * d;
    const float* kp = k + (g * 32) * stride + (int64_t)h * d + c;
    float vals[32];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        vals[j] = kp[j * stride];
        ss = ss + vals[j] * vals[j];
    }
    const float s = sqrtf(ss / 32.0f);
    const float t0 = cb.thr[0] * s, t1 = cb.thr[1] * s, t2 = cb.thr[2] * s;
    const bool live = s > 0.0f;
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float x = vals[j];
        uint32_t code = (x > t0 ? 1u : 0u) + (x > t1 ? 1u : 0u) + (x > t2 ? 1u : 0u);
        code = live ? code : 0u;
        if (j < 16) w0 |= code << (2 * j);
        else w1 |= code << (2 * (j - 16));
    }
    *reinterpret_cast<uint2*>(k_codes + gid * 8) = make_uint2(w0, w1);
    k_scale[gid] = f16_bits_rne(opaque(gain * s));   // round to f32, then to f16
}

// K append: one thread per (touched group, head, channel).  A group touched
// by an append is requantized from all of its cells present so far (cells
// [32g, min(32g + 32, n_end))): a whole group takes the RMS rule; a partial
// one is shrunk toward the previous group's scale, s = sqrtf((ss + (32 - n)
// prev^2) / 32) with prev = stored scale of group g-1 divided by the gain --
// read from k_scale when that group was completed by an earlier call,
// recomputed here (same sums, same order, same rounding) when this call
// touches it, so no thread reads a scale another thread of this launch
// writes; the first group, partial, takes sqrtf(ss / n).  Codes of absent
// cells are 0.
__device__ __forceinline__ void append_q2k_k_one(int64_t gid, const float* __restrict__ k, int64_t n_end,
                                                 int64_t g0, int n_kv, int d, float gain,
                                                 const Codebook4& cb, uint8_t* __restrict__ k_codes,
                                                 uint16_t* __restrict__ k_scale) {
    // gid = (g - g0, h, c)
    const int c = (int)(gid % d);
    const int64_t gh = gid / d;
    const int h = (int)(gh % n_kv);
    const int64_t g = g0 + gh / n_kv;
    const int64_t stride = (int64_t)n_kv * d;
    const int64_t hc = (int64_t)h * d + c;
    const int64_t rem = n_end - g * 32;
    const int n = rem < 32 ? (int)rem : 32;
    const float* kp = k + (g * 32) * stride + hc;
    float vals[32];
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        vals[j] = j < n ? kp[j * stride] : 0.0f;
        if (j < n) ss = ss + vals[j] * vals[j];
    }
    float s;
    if (n == 32) {
        s = sqrtf(ss / 32.0f);
    } else if (g == 0) {
        s = sqrtf(ss / (float)n);
    } else {
        uint16_t pbits;
        if (g - 1 < g0) {
            pbits = k_scale[(g - 1) * stride + hc];
        } else {
            const float* pp = k + ((g - 1) * 32) * stride + hc;
            float ps = 0.0f;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float x = pp[j * stride];
                ps = ps + x * x;
            }
            pbits = f16_bits_rne(opaque(gain * sqrtf(ps / 32.0f)));
        }
        const float prev = f16_bits_to_f32(pbits) / gain;
        const float fill = (float)(32 - n) * opaque(prev * prev);
        s = sqrtf(opaque(ss + fill) / 32.0f);
    }
    const float t0 = cb.thr[0] * s, t1 = cb.thr[1] * s, t2 = cb.thr[2] * s;
    const bool live = s > 0.0f;
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const float x = vals[j];
        uint32_t code = (x > t0 ? 1u : 0u) + (x > t1 ? 1u : 0u) + (x > t2 ? 1u : 0u);
        code = (live && j < n) ? code : 0u;
        if (j < 16) w0 |= code << (2 * j);
        else w1 |= code << (2 * (j - 16));
    }
    const int64_t o = g * stride + hc;
    *reinterpret_cast<uint2*>(k_codes + o * 8) = make_uint2(w0, w1);
    k_scale[o] = f16_bits_rne(opaque(gain * s));
}

// Overlay append (batch writer): one thread per (new cell, head, channel).
// Sinks go to their slots; of the other new cells only those among the last
// R = n_window + n_slack cells of the cache are written (ring slot n_sink +
// (c - n_sink) mod R), so no two threads write one slot and the result is
// what appending the cells one at a time would leave.
__device__ __forceinline__ void append_q2k_overlay_one(int64_t gid, const float* __restrict__ k,
                                                       const float* __restrict__ v, int64_t n_prev,
                                                       int64_t n_end, int n_kv, int d, int n_sink,
                                                       int n_window, int n_slack,
                                                       uint16_t* __restrict__ k_ovl,
                                                       uint16_t* __restrict__ v_ovl) {
    const int64_t per_cell = (int64_t)n_kv * d;
    const int64_t cell = n_prev + gid / per_cell;
    const int64_t hc = gid % per_cell;
    const int64_t R = (int64_t)n_window + n_slack;
    int64_t slot;
    if (cell < n_sink) slot = cell;
    else if (R > 0 && cell >= n_end - R) slot = n_sink + (cell - n_sink) % R;
    else return;
    k_ovl[slot * per_cell + hc] = f16_bits_rne(k[cell * per_cell + hc]);
    v_ovl[slot * per_cell + hc] = f16_bits_rne(v[cell * per_cell + hc]);
}

// V: one thread per 32-value block (q4_0: d = f16(amax/7), code = rint(x/d)+8).
__device__ __forceinline__ void encode_q2k_v_one(int64_t b, const float* __restrict__ v,
                                                 uint8_t* __restrict__ v_blocks) {
    const float* vp = v + b * 32;
    float vals[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j += 4) {
        const float4 a = *reinterpret_cast<const float4*>(vp + j);
        vals[j] = a.x; vals[j + 1] = a.y; vals[j + 2] = a.z; vals[j + 3] = a.w;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(vals[j]));
    const uint16_t dbits = f16_bits_rne(amax / 7.0f);
    const float df = f16_bits_to_f32(dbits);
    const bool zero = !(df != 0.0f);
    uint32_t code[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        float q = __builtin_rintf(vals[j] / (zero ? 1.0f : df)) + 8.0f;
        q = fminf(fmaxf(q, 0.0f), 15.0f);
        code[j] = zero ? 8u : (uint32_t)q;
    }
    uint16_t* out = reinterpret_cast<uint16_t*>(v_blocks + b * 18);   // 2-byte aligned
    out[0] = dbits;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
        const uint32_t lo = code[j] | (code[j + 16] << 4);
        const uint32_t hi = code[j + 1] | (code[j + 17] << 4);
        out[1 + j / 2] = (uint16_t)(lo | (hi << 8));
    }
}

// An append in one launch: the K groups it touches, the V blocks of its new
// cells and its overlay writes are independent (disjoint outputs; the K part
// reads a stored scale only for a group this launch does not write), so
// workgroups [0, nbk) run the K part, [nbk, nbk + nbv) the V part and the
// rest the overlay part.
__global__ __launch_bounds__(256) void k_append_q2k(const float* __restrict__ k, const float* __restrict__ v,
                                                    int64_t n_prev, int64_t n_end, int64_t g0, int64_t nk,
                                                    int64_t nbk, int64_t nb, int64_t nbv, int64_t no,
                                                    int n_kv, int d, float gain, Codebook4 cb, int n_sink,
                                                    int n_window, int n_slack, uint8_t* __restrict__ k_codes,
                                                    uint16_t* __restrict__ k_scale,
                                                    uint8_t* __restrict__ v_blocks,
                                                    uint16_t* __restrict__ k_ovl,
                                                    uint16_t* __restrict__ v_ovl) {
    const int64_t bx = blockIdx.x;
    if (bx < nbk) {
        const int64_t gid = bx * blockDim.x + threadIdx.x;
        if (gid < nk) append_q2k_k_one(gid, k, n_end, g0, n_kv, d, gain, cb, k_codes, k_scale);
    } else if (bx < nbk + nbv) {
        const int64_t b = (bx - nbk) * blockDim.x + threadIdx.x;
        if (b < nb) encode_q2k_v_one(b, v + n_prev * n_kv * d, v_blocks + n_prev * n_kv * (d / 32) * 18);
    } else {
        const int64_t gid = (bx - nbk - nbv) * blockDim.x + threadIdx.x;
        if (gid < no)
            append_q2k_overlay_one(gid, k, v, n_prev, n_end, n_kv, d, n_sink, n_window, n_slack, k_ovl, v_ovl);
    }
}

// Overlay of a whole cache (T cells): one thread per (slot, head, channel).
// Slot s < n_sink holds cell s; the other slots are a ring of R = n_window +
// n_slack: cell c >= n_sink lives in slot n_sink + (c - n_sink) mod R, and
// the slot holds the last cell of the cache mapped to it (the cell a
// one-at-a-time writer would have left there); slots no cell reaches are zero.
__device__ __forceinline__ void encode_q2k_overlay_one(int64_t gid, const float* __restrict__ k,
                                                       const float* __restrict__ v, int64_t T, int n_kv,
                                                       int d, int n_sink, int n_window, int n_slack,
                                                       uint16_t* __restrict__ k_ovl,
                                                       uint16_t* __restrict__ v_ovl) {
    const int64_t per_slot = (int64_t)n_kv * d;
    const int64_t R = (int64_t)n_window + n_slack;
    const int64_t slot = gid / per_slot;
    const int64_t hc = gid % per_slot;
    int64_t cell;
    if (slot < n_sink) {
        cell = slot < T ? slot : -1;
    } else {
        // largest c < T with c >= n_sink and (c - n_sink) mod R == slot - n_sink
        const int64_t base = T - 1 - slot;          // = (T-1) - n_sink - r
        cell = base < 0 ? -1 : T - 1 - base % R;
    }
    uint16_t kb = 0, vb = 0;
    if (cell >= 0) {
        kb = f16_bits_rne(k[cell * per_slot + hc]);
        vb = f16_bits_rne(v[cell * per_slot + hc]);
    }
    k_ovl[gid] = kb;
    v_ovl[gid] = vb;
}

// The whole-cache encoder in one launch: K groups, V blocks and overlay slots
// are independent, so workgroups [0, nbk) run the K part, [nbk, nbk + nbv)
// the V part and the rest the overlay part.
__global__ __launch_bounds__(256) void k_encode_q2k(const float* __restrict__ k, const float* __restrict__ v,
                                                    int64_t T, int64_t nk, int64_t nbk, int64_t nb,
                                                    int64_t nbv, int64_t no, int n_kv, int d, float gain,
                                                    Codebook4 cb, int n_sink, int n_window,
                                                    uint8_t* __restrict__ k_codes,
                                                    uint16_t* __restrict__ k_scale,
                                                    uint8_t* __restrict__ v_blocks,
                                                    uint16_t* __restrict__ k_ovl,
                                                    uint16_t* __restrict__ v_ovl) {
    const int64_t bx = blockIdx.x;
    if (bx < nbk) {
        const int64_t gid = bx * blockDim.x + threadIdx.x;
        if (gid < nk) encode_q2k_k_one(gid, k, n_kv, d, gain, cb, k_codes, k_scale);
    } else if (bx < nbk + nbv) {
        const int64_t b = (bx - nbk) * blockDim.x + threadIdx.x;
        if (b < nb) encode_q2k_v_one(b, v, v_blocks);
    } else {
        const int64_t gid = (bx - nbk - nbv) * blockDim.x + threadIdx.x;
        if (gid < no) encode_q2k_overlay_one(gid, k, v, T, n_kv, d, n_sink, n_window, 0, k_ovl, v_ovl);
    }
}

inline unsigned grid_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_encode_fp8(const float* x, int64_t n_rows, int32_t d, uint8_t* codes,
                             float* scales, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    const dim3 grid(grid_for(n_rows, kRowsPerBlock)), block(256);
    const bool vec_ok = (reinterpret_cast<uintptr_t>(x) % 16 == 0) &&
                        (reinterpret_cast<uintptr_t>(codes) % 8 == 0);
    if (d % 8 == 0 && d <= 4096 && vec_ok) {
        const int J = (d + 511) / 512;
        switch (J) {
            case 1: k_encode_fp8_vec<1><<<grid, block, 0, s>>>(x, n_rows, d, codes, scales); break;
            case 2: k_encode_fp8_vec<2><<<grid, block, 0, s>>>(x, n_rows, d, codes, scales); break;
            case 3:
            case 4: k_encode_fp8_vec<4><<<grid, block, 0, s>>>(x, n_rows, d, codes, scales); break;
            default: k_encode_fp8_vec<8><<<grid, block, 0, s>>>(x, n_rows, d, codes, scales); break;
        }
    } else {
        k_encode_fp8_any<<<grid, block, 0, s>>>(x, n_rows, d, codes, scales);
    }
    return hipGetLastError();
}

hipError_t launch_encode_tq4(const float* x, int64_t n_rows, int32_t d, uint64_t seed,
                             uint8_t* packed, float* radius, hipStream_t s) {
    if (n_rows == 0) return hipSuccess;
    const Codebook16 cb = codebook16();
    if (d == 512) {
        const bool wide = reinterpret_cast<uintptr_t>(packed) % 16 == 0;
        k_encode_tq4_512<<<grid_for(n_rows, kTq4RowsPerBlock512), 256, 0, s>>>(x, n_rows, seed, cb, packed,
                                                                               radius, wide);
        return hipGetLastError();
    }
    const dim3 grid(grid_for(n_rows, kRowsPerBlock)), block(256);
    const int E = d >= 64 ? d / 64 : 1;
    switch (E) {
        case 1: k_encode_tq4<1><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        case 2: k_encode_tq4<2><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        case 4: k_encode_tq4<4><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        case 8: k_encode_tq4<8><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        case 16: k_encode_tq4<16><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        case 32: k_encode_tq4<32><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        case 64: k_encode_tq4<64><<<grid, block, 0, s>>>(x, n_rows, d, seed, cb, packed, radius); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_encode_q2k(const float* k, const float* v, int64_t n_cells, int32_t n_kv,
                             int32_t d, float k_gain, int32_t n_sink, int32_t n_window,
                             uint8_t* k_codes, uint16_t* k_scale, uint8_t* v_blocks,
                             uint16_t* k_ovl, uint16_t* v_ovl, hipStream_t s) {
    const int64_t nk = n_cells / 32 * n_kv * d;             // K: (group, head, channel)
    const int64_t nb = n_cells * n_kv * (d / 32);           // V: q4_0 blocks
    const bool ovl = k_ovl != nullptr && n_sink + n_window > 0;
    const int64_t no = ovl ? (int64_t)(n_sink + n_window) * n_kv * d : 0;   // overlay slots
    const int64_t nbk = grid_for(nk, 256), nbv = grid_for(nb, 256), nbo = grid_for(no, 256);
    if (nbk + nbv + nbo == 0) return hipSuccess;
    k_encode_q2k<<<(unsigned)(nbk + nbv + nbo), 256, 0, s>>>(k, v, n_cells, nk, nbk, nb, nbv, no, n_kv, d,
                                                             k_gain, codebook4(), n_sink, n_window,
                                                             k_codes, k_scale, v_blocks, k_ovl, v_ovl);
    return hipGetLastError();
}

hipError_t launch_append_q2k(const float* k, const float* v, int64_t n_prev, int64_t n_new,
                             int32_t n_kv, int32_t d, float k_gain, int32_t n_sink,
                             int32_t n_window, int32_t n_slack, uint8_t* k_codes,
                             uint16_t* k_scale, uint8_t* v_blocks, uint16_t* k_ovl,
                             uint16_t* v_ovl, hipStream_t s) {
    if (n_new == 0) return hipSuccess;
    const int64_t n_end = n_prev + n_new;
    const int64_t g0 = n_prev / 32, g1 = (n_end + 31) / 32;
    const int64_t nk = (g1 - g0) * n_kv * d;                // K: touched (group, head, channel)
    const int64_t nb = n_new * n_kv * (d / 32);             // V: q4_0 blocks of the new cells
    const bool ovl = k_ovl != nullptr && n_sink + n_window > 0;
    const int64_t no = ovl ? n_new * n_kv * d : 0;          // overlay: (new cell, head, channel)
    const int64_t nbk = grid_for(nk, 256), nbv = grid_for(nb, 256), nbo = grid_for(no, 256);
    k_append_q2k<<<(unsigned)(nbk + nbv + nbo), 256, 0, s>>>(k, v, n_prev, n_end, g0, nk, nbk, nb, nbv, no,
                                                             n_kv, d, k_gain, codebook4(), n_sink,
                                                             n_window, n_slack, k_codes, k_scale,
                                                             v_blocks, k_ovl, v_ovl);
    return hipGetLastError();
}

}  // namespace kvq
