// Internal declarations shared by the translation units of libkvq.so.
// Device helpers are written for gfx950 (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/kvq.h"

namespace kvq {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Codebooks (computed once on the host, passed to kernels by value)
// ---------------------------------------------------------------------------
struct Codebook16 {
    float level[16];   // f16-rounded Lloyd-Max levels, ascending
    float thr[15];     // midpoints (level[k] + level[k+1]) / 2, exact in f32
};
struct Codebook4 {
    float level[4];
    float thr[3];
};
const Codebook16& codebook16();
const Codebook4& codebook4();

// ---------------------------------------------------------------------------
// Small device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t b) { return __builtin_bit_cast(float, b); }

// Pins x to a VGPR so the compiler cannot merge the operation that produced
// it with the one that consumes it (e.g. an f32 multiply followed by an
// f32->f16 conversion would otherwise become one v_fma_mix with a single
// rounding, which is not the two roundings the format defines).
__device__ __forceinline__ float opaque(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// IEEE binary16 bit pattern of x, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f16_bits_rne(float x) {
    _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// Value of an e4m3 byte times 2^-8 as an fp16 bit pattern.  Exact: e4m3's
// 4-bit exponent and 3-bit mantissa sit inside fp16's fields (its subnormals
// map to fp16 subnormals), so the rebias is a plain shift.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2_scaled(uint32_t two_bytes_lo16) {
    // input: byte0 in bits 0-7, byte1 in bits 8-15
    const uint32_t b0 = two_bytes_lo16 & 0xFFu, b1 = (two_bytes_lo16 >> 8) & 0xFFu;
    const uint32_t h0 = ((b0 & 0x80u) << 8) | ((b0 & 0x7Fu) << 7);
    const uint32_t h1 = ((b1 & 0x80u) << 8) | ((b1 & 0x7Fu) << 7);
    return h0 | (h1 << 16);
}

// e4m3 byte value as f32 (exact).  0x7F / 0xFF never occur in caches this
// library writes.
__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
    const uint32_t h = ((byte & 0x80u) << 8) | ((byte & 0x7Fu) << 7);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h) * 256.0f;
}

// Output `idx` (0-based) of SplitMix64 started from state `seed`: the
// generator is counter-based, output n mixes seed + (n+1) * golden gamma.
__device__ __forceinline__ uint64_t splitmix64_at(uint64_t seed, uint64_t idx) {
    uint64_t z = seed + (idx + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Value held by lane (l ^ M), M in {1, 2, 4, 8, 16, 32}, without an LDS round
// trip: DPP quad permutes for 1 and 2, DPP row shifts for 4 and 8 (lane l
// reads l + M or l - M inside its row of 16), v_permlane16/32_swap for 16 and
// 32 (a swap of v with itself leaves the own row / half in one result and
// the partner's in the other).
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    const int x = __builtin_bit_cast(int, v);
    const int lane = (int)(threadIdx.x & 63u);
    if constexpr (M == 1) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
    } else if constexpr (M == 2) {
        return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
    } else if constexpr (M == 4 || M == 8) {
        const int up = __builtin_amdgcn_mov_dpp(x, 0x100 + M, 0xF, 0xF, false);
        const int dn = __builtin_amdgcn_mov_dpp(x, 0x110 + M, 0xF, 0xF, false);
        return __builtin_bit_cast(float, (lane & M) ? dn : up);
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
        return __builtin_bit_cast(float, (lane & 16) ? r[0] : r[1]);
    } else {
        static_assert(M == 32, "xor_lane: M in {1, 2, 4, 8, 16, 32}");
        const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
        return __builtin_bit_cast(float, (lane & 32) ? r[0] : r[1]);
    }
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, xor_lane<32>(v));
    v = fmaxf(v, xor_lane<16>(v));
    v = fmaxf(v, xor_lane<8>(v));
    v = fmaxf(v, xor_lane<4>(v));
    v = fmaxf(v, xor_lane<2>(v));
    v = fmaxf(v, xor_lane<1>(v));
    return v;
}

// KV8 codes.  [colibri #399] "Summary" / "Commits" item 1: e4m3, round to
// nearest even, row scale s = fl(amax/448).
// A quotient is an element divided by its row's scale s.  While
// s is a normal float the quotient is at most 448 (1 + 2^-23) in magnitude and
// rounds to at most 448.  A row whose amax is below about 2^-126 * 448 has a
// subnormal scale, coarse enough that quotients reach about 672 (for amax
// near 2^-149 * 448 * 1.5); those saturate to 448 (0x7E / 0xFE), so every
// quotient is clamped to [-448, 448] before the conversion, which is not
// relied on to saturate.  The clamp returns its input unchanged inside the
// range (-0.0 included), so it leaves every other byte as it was.
__device__ __forceinline__ float sat448(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Four f32 quotients -> four e4m3 bytes with the hardware conversion (OCP
// e4m3fn, round to nearest even, sign kept on a zero result).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), lo, true);
}

// ---------------------------------------------------------------------------
// Launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
hipError_t launch_encode_fp8(const float* x, int64_t n_rows, int32_t d, uint8_t* codes,
                             float* scales, hipStream_t s);
hipError_t launch_encode_tq4(const float* x, int64_t n_rows, int32_t d, uint64_t seed,
                             uint8_t* packed, float* radius, hipStream_t s);
hipError_t launch_encode_q2k(const float* k, const float* v, int64_t n_cells, int32_t n_kv,
                             int32_t d, float k_gain, int32_t n_sink, int32_t n_window,
                             uint8_t* k_codes, uint16_t* k_scale, uint8_t* v_blocks,
                             uint16_t* k_ovl, uint16_t* v_ovl, hipStream_t s);
hipError_t launch_append_q2k(const float* k, const float* v, int64_t n_prev, int64_t n_new,
                             int32_t n_kv, int32_t d, float k_gain, int32_t n_sink,
                             int32_t n_window, int32_t n_slack, uint8_t* k_codes,
                             uint16_t* k_scale, uint8_t* v_blocks, uint16_t* k_ovl,
                             uint16_t* v_ovl, hipStream_t s);

// Attention plan: how the rows are split and what the workspace holds.
struct AttnPlan {
    int32_t path;          // 0: general f32 path, 1: MFMA latent (KV8/TQ4), 2: MFMA q2k
    int32_t log2_domain;   // partial maxima m are in log2 units (else natural log)
    int32_t n_qrows;       // S * Hq query rows
    int32_t heads_per_blk; // query rows handled by one workgroup
    int32_t n_qgroups;     // workgroups along the query-row axis
    int32_t n_split;       // chunks along T
    int64_t chunk;         // rows per chunk
    size_t ws_bytes;       // partials: n_split * n_qrows * (d + 2) floats
};
// q may be NULL when only sizing the workspace (the plan then assumes an
// aligned query; a misaligned one gets a plan with a larger-or-equal workspace)
// wide_decode = false keeps a decode on the per-head-group kernel (whose
// partials are 4x smaller: the no-allocation entry point's scratch)
AttnPlan make_plan(const kvq_cache& kv, int32_t Hq, int32_t S, const void* q, bool wide_decode = true);

// Raise a kernel's dynamic LDS limit to `bytes` once per device: the first
// launch on a device sets it, later launches skip the runtime call.  `done`
// is one static mask per kernel (bit = device ordinal; ordinals past 63 set it
// every time).
inline hipError_t set_dyn_lds_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
    return e;
}
AttnPlan generic_plan(const kvq_cache& kv, int32_t Hq, int32_t S);

// A decode step's new KV8 row: f32 x [d], encoded into row `row` of the
// cache whose codes / scales these are (the same buffers as the kvq_cache's)
struct NewRow {
    const float* x;
    uint8_t* codes;
    float* scales;
    int64_t row;
};

// MFMA decode for the fp8 MLA latent (d = 512, heads in groups of 16)
bool mla_mfma_eligible(const kvq_cache& kv, int32_t Hq, int32_t S, const void* q);
void mla_mfma_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p, bool wide_decode = true);
// whether launch_mla_mfma can encode nr's row inside the decode launch
bool mla_append_fusable(const kvq_cache& kv, const AttnPlan& p, int32_t Hq, int32_t S, int64_t pos0,
                        const int32_t* idx, const NewRow* nr);
// with p.n_split == 1 it writes out / lse itself (out unrotated for TQ4: run
// launch_unrotate after it).  idx != NULL (decode only): kv.n_rows is the
// length of the row list idx, whose entries name rows of a cache of n_cache
// rows; entries outside [0, n_cache) are skipped.  nr != NULL: the new row is
// encoded and written by the decode launch itself (only where
// mla_append_fusable holds).
hipError_t launch_mla_mfma(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                           int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                           float* part_ml, float* out, float* lse, hipStream_t s,
                           const int32_t* idx = nullptr, int64_t n_cache = 0,
                           const NewRow* nr = nullptr);
// KV8 prefill (S >= 8): flash-attention tiles shared by 4 tokens, split into
// chunks (partials for the combine) unless one chunk fills the GPU (then
// out / lse directly)
bool mla_prefill_kv8_eligible(const kvq_cache& kv, int32_t Hq, int32_t S);
void mla_prefill_kv8_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p);
hipError_t launch_mla_prefill_kv8(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                                  int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                                  float* part_ml, float* out, float* lse, hipStream_t s);
// TQ4 decode of one token with 64 heads over a long cache (the same shared
// tiles: a workgroup takes the 4 head groups of a chunk, so each row is
// decoded once).  Its plan has heads_per_blk = 64; a launch with pos0 >= 0 or
// a row list runs the per-head-group kernel on the same plan.
bool mla_decode64_eligible(const kvq_cache& kv, int32_t Hq, int32_t S);
void mla_decode64_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p);
hipError_t launch_mla_decode64(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq, int32_t S,
                               int64_t pos0, float sm_scale, float* part_acc, float* part_ml, float* out,
                               float* lse, hipStream_t s);
// MFMA GQA decode for q2k caches (d = 256, 8 query heads per KV head)
bool q2k_mfma_eligible(const kvq_cache& kv, int32_t Hq, int32_t S, const void* q);
void q2k_mfma_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p);
// S query tokens (token s attends cells t <= pos0 + s; pos0 < 0 with S = 1:
// every cell).  Launches the decode over the bulk cells and its combine
// (which also attends the overlay cells), writing out / lse.
hipError_t launch_q2k_mfma(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                           int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                           float* part_ml, float* out, float* lse, hipStream_t s);
// chunk merge (and TQ4 unrotation) shared by the attention paths
// TQ4: out_h <- D H out_h for every query row (the combine step's rotation)
hipError_t launch_unrotate(float* out, int64_t n_qrows, int d, uint64_t seed, hipStream_t s);
hipError_t launch_combine(int32_t fmt, const float* part_acc, const float* part_ml, int n_split,
                          int64_t n_qrows, int d, uint64_t seed, bool log2_domain, float* out,
                          float* lse, hipStream_t s);

// The argument checks of attn_decode_quant (all but the workspace) and, when
// they pass, the plan of the request.
kvq_status decode_request(const kvq_cache* kv, const float* q, int32_t n_q_heads, const float* out,
                          const float* lse, AttnPlan& plan);

// idx / n_cache: row list of a gather decode (plan path 1 only), as for
// launch_mla_mfma
// nr != NULL (KV8): the step's new row is encoded into the cache first, by
// the decode launch itself where mla_append_fusable holds, else by the KV8
// encoder launched before it.
hipError_t launch_attention(const kvq_cache& kv, const AttnPlan& plan, const float* q,
                            int32_t S, int32_t Hq, int64_t pos0, float sm_scale, float* out,
                            float* lse, void* ws, hipStream_t s, const int32_t* idx = nullptr,
                            int64_t n_cache = 0, const NewRow* nr = nullptr);

}  // namespace kvq
