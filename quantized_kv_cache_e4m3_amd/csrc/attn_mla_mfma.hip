// Decode and chunked-prefill attention for the MLA latent (d = 512, heads in
// groups of 16) on the gfx950 matrix cores, over KV8 rows (fp8 e4m3 values +
// f32 row scale) and TQ4 rows (4-bit codebook indices + f32 radius).
//
// [colibri #553] "What's in it" / [colibri #399] "Commits" item 2: the rows
// are consumed as they are stored, split over T with a combine step, and the
// latent row is both key and value.  KV8: the e4m3 values enter the dot
// products, the row scale stays outside.  TQ4 ([colibri #553] "What's in it",
// "Ready for review" comment): the query is rotated once per head (q' = H D q),
// the scores are (r/n) q'.c with c the codebook values, the context is
// accumulated in the rotated domain and unrotated once in the combine step.
//
// With 64 heads sharing every row the decode is a dense contraction (4*H*d
// flops per row), so both products run on MFMA v_mfma_f32_16x16x32_f16:
//   scores   S^T[row, head] = K[row, :] . Q[head, :]       (A = K, B = Q^T)
//   context  C[head, dim]  += P[head, row] . V[row, dim]   (A = P, B = V)
// e4m3 values and the fp16-rounded codebook levels are exact in f16, so K and
// V are exact operands.  The f32 side (the query, and the weights p * row
// factor) is split into an f16 high part and an f16 residual and multiplied
// twice, which keeps the products to ~2^-22 relative error; both are
// pre-scaled by powers of two (exact) so the residual never underflows.
//
// Work layout.  Workgroup = (chunk of rows, group of 16 heads), 8 waves = 4
// pairs; pair p takes 32-row tiles p, p+4, ... of the chunk.  The two waves of
// a pair split the latent width: wave half h owns dims [256h, 256h+256) for
// both the score partial and the context, so each wave keeps only 64 VGPRs of
// query and 64 of accumulator (two waves fit per SIMD) and reads only the
// half-rows it loaded itself.  Per tile a wave prefetches its next half-rows
// into registers, stores the current ones into its private LDS tile (rows
// padded by 16 bytes: row reads and transpose reads with immediate offsets
// stay bank-conflict free), adds its partner's partial scores through LDS
// (one barrier), runs the online softmax on the full scores (both waves
// compute identical values), and accumulates its context half.  Score tile 0
// holds rows 0..15, tile 1 rows 16..31; the score MFMA output is then already
// the context MFMA's A operand for the row order rho(g, e) = 16*(e/4) + 4g +
// e%4, and the V operand (8 rows of one dim per lane) comes from
// ds_read_b64_tr_b8 with source rows in that same order.
//
// Operand decode.  KV8: v_cvt_scalef32_pk_f16_fp8 (exact), for the K operand
// from the wave's LDS rows and for the V operand after ds_read_b64_tr_b8.
// TQ4: a 256-entry LDS table maps one packed byte to the two f16 levels of its
// nibbles; K operands take 4 lookups per 8 dims, straight from the prefetch
// registers (a lane's k-steps cover dims 64u + 16g + [0, 8) and [8, 16), the
// query is permuted to match).  The decoded rows are also written to the
// wave's LDS tile as f16, and the context reads its V operands from there
// with ds_read_b64_tr_b16, so every nibble is decoded once.
//
// Rope part of the key ([colibri #553] rebase comment, item 1: the kv_lora
// and qk_rope parts of an MLA row are quantized separately).  With a 64-wide
// rope part the key is [latent | rope] and the value the latent alone: each
// wave adds one more score k-step (its 32 rope dims, operands loaded straight
// in the MFMA layout, TQ4 decoded through the same byte table), the query's
// rope part is staged once (TQ4: rotated with the rope seed), and since the
// two parts have different row factors each wave scales its partial scores
// before the partner exchange.
//
// Decode step with a new row ([colibri #399] "Summary" / "Commits" item 1 for
// the producer): the append variant encodes the step's new KV8 row in the
// workgroups whose chunk holds it, with the encoder's own conversion, and
// takes its codes and scale from registers wherever the loads read that row
// (LDS tile row, row factors, pre-scale maximum); one workgroup writes it to
// the cache.  No workgroup reads the row back, so nothing waits on the write.
//
// Scores are kept in log2 units (exp2 on the hardware transcendental unit).
// Online softmax keeps one running max per head and rescales only when the
// max grows by more than 8 (p <= 2^8, weights pre-scaled to stay in f16 range).  The 4
// pairs merge in LDS and write one (m, l, acc) partial per chunk (m in log2
// units); the combine kernel merges the chunks.  With a single chunk (a long
// prefill) the workgroup writes the normalized output and lse itself.
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 512;
constexpr int DR = 64;                  // rope part of the key (when present)
constexpr int HALF = D / 2;             // dims per wave
constexpr int KSTEPS = HALF / 32;       // 8 score k-steps per wave
constexpr int NT = HALF / 16;           // 16 context dim tiles per wave
constexpr int TR = 32;                  // rows per tile
constexpr int kWaves = 8, kPairs = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int MROW = D + 4;            // merge row stride (floats): heads 4 apart land in different banks
constexpr int kMergeLds = kPairs * 16 * MROW * 4;
constexpr int QROW = 2 * D + 16;        // LDS bytes per staged query half-row (f16, padded)
// Lazy rescale: the running max used for the weights moves only when the
// true max exceeds it by more than kRescaleSlack (log2 units), so p <= 2^8.
// The weight pre-scale puts 2^ew * (max row factor) in [2^6, 2^7), so every
// weight p * factor * 2^ew stays below 2^15 (f16 range), and a weight with
// p near 1 still has a normal f16 residual (about 22 significant bits).
constexpr float kRescaleSlack = 8.0f;
constexpr int kWeightShift = 7;         // 2^(14 - 7) headroom bound, see above
constexpr float kLog2e = 1.4426950408889634f;
constexpr int64_t kMaxChunk = int64_t{1} << 21;   // rows per workgroup chunk (1 GiB of KV8 rows)

// Per-format layout.  KV8: a wave's half-tile is 32 rows x HB bytes of fp8,
// loaded as NLD 16-byte pieces per lane (lane i, load k -> row RPL*k + i/LPR,
// piece i%LPR) and stored as is; LDR is the padded LDS row stride.  TQ4: the
// half-tile's nibbles are loaded in the K operand's own layout (lane (n16, g):
// 8 bytes at 32u + 8g of rows n16 and 16 + n16), decoded once through the
// byte table, and the decoded f16 rows are stored (LDR = f16 row stride) for
// the context's transpose reads.  The partner exchange is double-buffered for
// KV8 and single-buffered (a second barrier per tile) for TQ4, whose f16
// tiles fill the LDS.
template <int FMT> struct Fmt;
template <> struct Fmt<KVQ_FP8> {
    static constexpr int ROWB = D, HB = HALF, LDR = HB + 16, LPR = HB / 16, RPL = 64 / LPR;
    static constexpr int NLD = TR / RPL;
    static constexpr int LOG2_ROW_DIV = 0;      // row factor = scale
    static constexpr int EXCH_BUFS = 2;
};
template <> struct Fmt<KVQ_TQ4> {
    static constexpr int ROWB = D / 2, HB = HALF / 2, LDR = 2 * HALF + 16;
    static constexpr int LOG2_ROW_DIV = 9;      // row factor = radius / 512
    static constexpr int EXCH_BUFS = 1;
};
template <int FMT>
constexpr int tile_lds() {
    return kWaves * TR * Fmt<FMT>::LDR + Fmt<FMT>::EXCH_BUFS * kWaves * 512 * 4;
}
// KV8 stages the query above its tiles (no barrier between the staging reads
// and the first tile store); TQ4's tiles leave no room, so it stages at 0
template <int FMT>
constexpr int q_stage_off() { return FMT == KVQ_FP8 ? tile_lds<FMT>() : 0; }
template <int FMT>
constexpr int q_stage_end() { return q_stage_off<FMT>() + 16 * 2 * (2 * D + 16); }
template <int FMT>
constexpr int dyn_lds() {
    const int a = tile_lds<FMT>() > kMergeLds ? tile_lds<FMT>() : kMergeLds;
    return a > q_stage_end<FMT>() ? a : q_stage_end<FMT>();
}

struct MlaArgs {
    const uint8_t* codes;
    const float* scales;    // KV8: row scale; TQ4: radius
    const float* q;         // [S][Hq][D]
    float sm_scale;
    int64_t T;
    int32_t Hq;
    int32_t S;              // query tokens (1: decode)
    int64_t pos0;           // prefill: position of token 0; < 0: decode (all T rows)
    int64_t chunk;          // rows per workgroup chunk (multiple of 128)
    int32_t xcd_map;        // 1: keep the head groups of a chunk on one XCD
    float* part_acc;        // [n_chunks][S*Hq][D]
    float* part_ml;         // [n_chunks][S*Hq][2]
    int32_t direct;         // one chunk: write out / lse here, no partials
    float* out;             // [S*Hq][D] (direct)
    float* lse;             // [S*Hq] or null (direct)
    uint64_t seed;          // TQ4 rotation seed
    float level[16];        // TQ4 codebook (fp16 values)
    const int32_t* idx;     // gather: logical row t reads cache row idx[t] (T = list length); null: t
    int64_t n_cache;        // gather: cache rows (an index outside [0, n_cache) is skipped)
    const uint8_t* rcodes;  // rope rows: KV8 [.][64], TQ4 [.][32] (rope variant only)
    const float* rscales;   // rope row scale / radius
    uint64_t rseed;         // TQ4 rope rotation seed
    // append variant (KV8): the step's new row x_new, f32 [D], is encoded by
    // the workgroups whose chunk holds cache row new_row and written there
    const float* x_new;
    uint8_t* new_codes;     // the cache's codes of row new_row
    float* new_scale;       // the cache's scale of row new_row
    int64_t new_row;
};

__device__ __forceinline__ half8_t cvt8(uint32_t lo, uint32_t hi) {
    const half2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const half2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const half2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    half8_t r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
}

// 8 nibbles (4 bytes, low nibble first) -> 8 f16 levels via the byte table
__device__ __forceinline__ half8_t lut8(const uint32_t* lut, uint32_t x) {
    u32x4 r;
    r[0] = lut[x & 0xFFu];
    r[1] = lut[(x >> 8) & 0xFFu];
    r[2] = lut[(x >> 16) & 0xFFu];
    r[3] = lut[x >> 24];
    return __builtin_bit_cast(half8_t, r);
}

// power-of-two exponent e with x * 2^e in [2^13, 2^14) (0 for x == 0)
__device__ __forceinline__ int headroom_exp(float x) {
    if (!(x > 0.0f)) return 0;
    int k;
    (void)frexpf(x, &k);
    return 14 - k;
}

// row of the tile held in context slot e of lane group g
__device__ __forceinline__ int rho(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

// query dims (within the wave's half) of k-step s for lane group g
template <int FMT>
__device__ __forceinline__ int q_dim(int s, int g) {
    if constexpr (FMT == KVQ_FP8) return 32 * s + 8 * g;
    else return 64 * (s >> 1) + 16 * g + 8 * (s & 1);
}

// prefetched half-tile of a wave plus the row factors of its context rows
// (listed rows: s[0] alone, the factor of tile row lane % 32, read through
// row_factor as for the rope part)
template <int FMT> struct PfRegs;
template <> struct PfRegs<KVQ_FP8> {
    u32x4 v[Fmt<KVQ_FP8>::NLD];
    float s[8];                 // gather: -0.0 marks a padding entry (stored factors are >= +0)
};
template <> struct PfRegs<KVQ_TQ4> {
    uint2 v[2][KSTEPS / 2];     // [row tile][u]: bytes 32u + 8g .. +8 of row 16*rt + n16
    float s[8];
};

template <bool GATHER, int FMT>
__device__ __forceinline__ float row_factor(const PfRegs<FMT>& r, int g, int e) {
    if constexpr (GATHER) return __shfl(r.s[0], rho(g, e));
    else return r.s[e];
}

// gather helpers: the list entry of tile row lane % 32 (rows past T repeat
// entry T-1), and the cache row an entry reads (row 0 for an entry outside
// the cache: in bounds, masked later)
__device__ __forceinline__ int32_t tile_entry(const int32_t* idx, int64_t row0, int64_t T, int lane) {
    int64_t t = row0 + (lane & 31);
    t = t < T ? t : T - 1;
    return idx[t];
}
__device__ __forceinline__ int64_t listed_row(int32_t ent, int64_t n_cache) {
    return (ent >= 0 && ent < n_cache) ? (int64_t)ent : 0;
}

// prefetch of one half-tile plus the row factors of this lane's context rows
// rho(g, 0..7).  Tiles that reach past T clamp their rows to T-1 (in bounds;
// masked later).
template <int FMT>
__device__ __forceinline__ void prefetch(PfRegs<FMT>& r, const uint8_t* codes, const float* scales,
                                         int64_t row0, int64_t T, int half, int lane, int g,
                                         const int32_t* idx, int64_t n_cache) {
    using F = Fmt<FMT>;
    if (idx != nullptr) {
        // gather: one list entry per lane (tile row lane % 32), shared by
        // shuffles; then every load is issued unconditionally (an entry
        // outside the cache reads row 0) and masked afterwards, so the loads
        // stay in flight together
        const int32_t mine = tile_entry(idx, row0, T, lane);
        if constexpr (FMT == KVQ_FP8) {
            const int r_in = lane / F::LPR, piece = lane % F::LPR;
#pragma unroll
            for (int k = 0; k < F::NLD; ++k) {
                const int64_t pr = listed_row(__shfl(mine, F::RPL * k + r_in), n_cache);
                r.v[k] = *reinterpret_cast<const u32x4*>(codes + pr * F::ROWB + F::HB * half + 16 * piece);
            }
        } else {
            const int n16 = lane & 15;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int64_t pr = listed_row(__shfl(mine, 16 * rt + n16), n_cache);
                const uint8_t* base = codes + pr * F::ROWB + F::HB * half + 8 * g;
#pragma unroll
                for (int u = 0; u < KSTEPS / 2; ++u) r.v[rt][u] = *reinterpret_cast<const uint2*>(base + 32 * u);
            }
        }
        const bool valid = mine >= 0 && mine < n_cache;
        const float f = scales[listed_row(mine, n_cache)];
        asm volatile("" ::: "memory");
        // a padding entry's factor becomes -0.0: its weight is zero and the
        // softmax masks its score (stored row factors are never negative)
        r.s[0] = valid ? f : -0.0f;
        return;
    }
    const bool full = row0 + TR <= T;
    if constexpr (FMT == KVQ_FP8) {
        const int r_in = lane / F::LPR, piece = lane % F::LPR;
        if (full) {
            const uint8_t* base = codes + (row0 + r_in) * F::ROWB + F::HB * half + 16 * piece;
#pragma unroll
            for (int k = 0; k < F::NLD; ++k)
                r.v[k] = *reinterpret_cast<const u32x4*>(base + (int64_t)F::RPL * k * F::ROWB);
        } else {
#pragma unroll
            for (int k = 0; k < F::NLD; ++k) {
                int64_t t = row0 + F::RPL * k + r_in;
                t = t < T ? t : T - 1;
                r.v[k] = *reinterpret_cast<const u32x4*>(codes + t * F::ROWB + F::HB * half + 16 * piece);
            }
        }
    } else {
        const int n16 = lane & 15;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            int64_t t = row0 + 16 * rt + n16;
            t = t < T ? t : T - 1;
            const uint8_t* base = codes + t * F::ROWB + F::HB * half + 8 * g;
#pragma unroll
            for (int u = 0; u < KSTEPS / 2; ++u) r.v[rt][u] = *reinterpret_cast<const uint2*>(base + 32 * u);
        }
    }
    if (full) {
        const float4 s0 = *reinterpret_cast<const float4*>(scales + row0 + 4 * g);
        const float4 s1 = *reinterpret_cast<const float4*>(scales + row0 + 16 + 4 * g);
        r.s[0] = s0.x; r.s[1] = s0.y; r.s[2] = s0.z; r.s[3] = s0.w;
        r.s[4] = s1.x; r.s[5] = s1.y; r.s[6] = s1.z; r.s[7] = s1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int64_t t = row0 + rho(g, e);
            t = t < T ? t : T - 1;
            r.s[e] = scales[t];
        }
    }
}

// Dense rows are read through two buffer resources per workgroup (codes and
// row factors) whose base is the chunk's first row and whose range ends at
// the chunk's last attended row.  A load past the range returns zeros without
// touching memory, so tiles that reach past the chunk (the ragged last tile,
// the prefetch after the last tile) need no per-row clamping, and every
// offset is a 32-bit row offset inside the chunk.
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 (32-bit data format)
struct ChunkBufs {
    __amdgpu_buffer_rsrc_t codes, scales;
};

template <int FMT>
__device__ __forceinline__ ChunkBufs chunk_bufs(const uint8_t* codes, const float* scales, int64_t c0,
                                                int n_rows) {
    using F = Fmt<FMT>;
    const int rows = n_rows > 0 ? n_rows : 0;
    ChunkBufs b;
    b.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes + c0 * F::ROWB), (short)0,
                                                rows * F::ROWB, kBufWord3);
    b.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(scales + c0), (short)0, rows * 4,
                                                 kBufWord3);
    return b;
}

// prefetch() for dense rows: rel_row0 is the tile's first row in the chunk
template <int FMT>
__device__ __forceinline__ void prefetch_dense(PfRegs<FMT>& r, const ChunkBufs& b, int rel_row0, int half,
                                               int lane, int g) {
    using F = Fmt<FMT>;
    if constexpr (FMT == KVQ_FP8) {
        const int r_in = lane / F::LPR, piece = lane % F::LPR;
        const int off = (rel_row0 + r_in) * F::ROWB + F::HB * half + 16 * piece;
#pragma unroll
        for (int k = 0; k < F::NLD; ++k)
            r.v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   b.codes, off + F::RPL * k * F::ROWB, 0, 0));
    } else {
        const int n16 = lane & 15;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int off = (rel_row0 + 16 * rt + n16) * F::ROWB + F::HB * half + 8 * g;
#pragma unroll
            for (int u = 0; u < KSTEPS / 2; ++u)
                r.v[rt][u] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(b.codes, off + 32 * u, 0, 0));
        }
    }
    const int soff = (rel_row0 + 4 * g) * 4;
    const f32x4 s0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.scales, soff, 0, 0));
    const f32x4 s1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.scales, soff + 64, 0, 0));
    r.s[0] = s0[0]; r.s[1] = s0[1]; r.s[2] = s0[2]; r.s[3] = s0[3];
    r.s[4] = s1[0]; r.s[5] = s1[1]; r.s[6] = s1[2]; r.s[7] = s1[3];
}

// prefetched rope operands of a wave: its 32 rope dims (32*half + 8g .. +8)
// of rows 16*rt + n16, in the score A operand's layout, plus the rope row
// factors of rows rho(g, 0..7).  Listed rows: s[0] alone holds the factor of
// tile row lane % 32 (0 for a padding entry), one load per lane, and the
// consumer reads rho(g, e)'s by a lane shuffle (rope_factor): eight gathered
// addresses fewer in flight.
template <int FMT> struct RopeRegs;
template <> struct RopeRegs<KVQ_FP8> {
    uint2 v[2];                 // 8 e4m3 codes
    float s[8];
};
template <> struct RopeRegs<KVQ_TQ4> {
    uint32_t v[2];              // 8 nibbles
    float s[8];
};

template <bool GATHER, int FMT>
__device__ __forceinline__ float rope_factor(const RopeRegs<FMT>& r, int g, int e) {
    if constexpr (GATHER) return __shfl(r.s[0], rho(g, e));
    else return r.s[e];
}

template <int FMT>
__device__ __forceinline__ void prefetch_rope(RopeRegs<FMT>& r, const uint8_t* rcodes,
                                              const float* rscales, int64_t row0, int64_t T,
                                              int half, int n16, int g, const int32_t* idx,
                                              int64_t n_cache) {
    if (idx != nullptr) {
        // gather: as in prefetch(), one list entry per lane shared by shuffles
        const int lane = 16 * g + n16;
        const int32_t mine = tile_entry(idx, row0, T, lane);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int64_t pr = listed_row(__shfl(mine, 16 * rt + n16), n_cache);
            if constexpr (FMT == KVQ_FP8)
                r.v[rt] = *reinterpret_cast<const uint2*>(rcodes + pr * DR + 32 * half + 8 * g);
            else
                r.v[rt] = *reinterpret_cast<const uint32_t*>(rcodes + pr * (DR / 2) + 16 * half + 4 * g);
        }
        const bool valid = mine >= 0 && mine < n_cache;
        const float f = rscales[listed_row(mine, n_cache)];
        asm volatile("" ::: "memory");
        r.s[0] = valid ? f : 0.0f;
        return;
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        int64_t t = row0 + 16 * rt + n16;
        t = t < T ? t : T - 1;
        if constexpr (FMT == KVQ_FP8)
            r.v[rt] = *reinterpret_cast<const uint2*>(rcodes + t * DR + 32 * half + 8 * g);
        else
            r.v[rt] = *reinterpret_cast<const uint32_t*>(rcodes + t * (DR / 2) + 16 * half + 4 * g);
    }
    if (row0 + TR <= T) {
        const float4 s0 = *reinterpret_cast<const float4*>(rscales + row0 + 4 * g);
        const float4 s1 = *reinterpret_cast<const float4*>(rscales + row0 + 16 + 4 * g);
        r.s[0] = s0.x; r.s[1] = s0.y; r.s[2] = s0.z; r.s[3] = s0.w;
        r.s[4] = s1.x; r.s[5] = s1.y; r.s[6] = s1.z; r.s[7] = s1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int64_t t = row0 + rho(g, e);
            t = t < T ? t : T - 1;
            r.s[e] = rscales[t];
        }
    }
}

// prefetch_rope() for dense rows, through the rope part's own buffer
// resources (same chunk base and range as the latent rows)
template <int FMT>
__device__ __forceinline__ void prefetch_rope_dense(RopeRegs<FMT>& r, const ChunkBufs& b, int rel_row0,
                                                    int half, int n16, int g) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int row = rel_row0 + 16 * rt + n16;
        if constexpr (FMT == KVQ_FP8)
            r.v[rt] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                                                    b.codes, row * DR + 32 * half + 8 * g, 0, 0));
        else
            r.v[rt] = __builtin_amdgcn_raw_buffer_load_b32(b.codes, row * (DR / 2) + 16 * half + 4 * g, 0, 0);
    }
    const int soff = (rel_row0 + 4 * g) * 4;
    const f32x4 s0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.scales, soff, 0, 0));
    const f32x4 s1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.scales, soff + 64, 0, 0));
    r.s[0] = s0[0]; r.s[1] = s0[1]; r.s[2] = s0[2]; r.s[3] = s0[3];
    r.s[4] = s1[0]; r.s[5] = s1[1]; r.s[6] = s1[2]; r.s[7] = s1[3];
}

template <int FMT, bool ROPE, bool GATHER, bool APPEND>
__global__ __launch_bounds__(kThreads, 1) void k_mla_mfma(MlaArgs a) {
    using F = Fmt<FMT>;
    static_assert(!APPEND || (FMT == KVQ_FP8 && !ROPE && !GATHER), "append: dense KV8 rows only");
    // the row list (top-k gather); a compile-time null in the dense variants,
    // which then carry none of the gather code
    const int32_t* const idx = GATHER ? a.idx : nullptr;
    constexpr int QW = ROPE ? D + DR : D;               // query row width (latent | rope)
    constexpr int LDR = F::LDR;
    constexpr int TILE_BYTES = TR * LDR;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float ml_s[kPairs][16][2];
    __shared__ float red_s[kWaves];
    __shared__ uint32_t lut_s[FMT == KVQ_TQ4 ? 256 : 1];
    // rope query part per head: f16 high part then residual, 64 dims each
    __shared__ __attribute__((aligned(16))) _Float16 qr_s[ROPE ? 16 * 2 * DR : 8];
    __shared__ float qrs_s[16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1, half = wave & 1;
    const int g = lane >> 4, n16 = lane & 15;
    const int n_hg = (a.Hq + 15) / 16;                     // the last group may hold fewer heads
    int b = blockIdx.x;
    if (a.xcd_map) b = (b & 7) * (gridDim.x >> 3) + (b >> 3);
    const int per_tok = gridDim.x / a.S;                    // n_split * n_hg
    const int tok = b / per_tok;
    const int chunk = (b % per_tok) / n_hg, hg = b % n_hg;
    const int64_t lim = a.pos0 < 0 ? a.T : a.pos0 + tok + 1;   // causal limit of this token
    const int64_t n_qrows = (int64_t)a.S * a.Hq;
    const int64_t qrow0 = (int64_t)tok * a.Hq + hg * 16;    // first query row of this workgroup
    const int hv = (a.Hq - hg * 16 < 16) ? a.Hq - hg * 16 : 16;   // its heads; the rest are zero queries
    const int64_t c0 = (int64_t)chunk * a.chunk;
    const int64_t c1 = (c0 + a.chunk < lim) ? c0 + a.chunk : lim;
    const int64_t n_rows = c1 - c0;
    const int n_tiles = n_rows > 0 ? (int)((n_rows + TR - 1) / TR) : 0;
    const int n_iter = (n_tiles + kPairs - 1) / kPairs;      // same for every wave (barriers)

    uint8_t* tile = lds + wave * TILE_BYTES;
    float* exch = reinterpret_cast<float*>(lds + kWaves * TILE_BYTES);

    // first half-tile in flight while the query is staged
    // rows of the chunk (< 2^31 / row bytes: the launch plan caps the chunk)
    const int n_rows32 = n_rows > 0 ? (int)n_rows : 0;
    ChunkBufs cbuf;
    if constexpr (!GATHER) cbuf = chunk_bufs<FMT>(a.codes, a.scales, c0, n_rows32);
    PfRegs<FMT> pf;
    if constexpr (GATHER)
        prefetch<FMT>(pf, a.codes, a.scales, c0 + (int64_t)pair * TR, a.T, half, lane, g, idx, a.n_cache);
    else
        prefetch_dense<FMT>(pf, cbuf, pair * TR, half, lane, g);
    RopeRegs<FMT> rpf;
    ChunkBufs rbuf;
    if constexpr (ROPE && !GATHER) {
        constexpr int RB = FMT == KVQ_FP8 ? DR : DR / 2;           // rope row bytes
        rbuf.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.rcodes + c0 * RB), (short)0,
                                                       n_rows32 * RB, kBufWord3);
        rbuf.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.rscales + c0), (short)0,
                                                        n_rows32 * 4, kBufWord3);
        prefetch_rope_dense<FMT>(rpf, rbuf, pair * TR, half, n16, g);
    } else if constexpr (ROPE) {
        prefetch_rope<FMT>(rpf, a.rcodes, a.rscales, c0 + (int64_t)pair * TR, a.T, half, n16, g,
                           idx, a.n_cache);
    }

    // dense chunks of more than one tile per pair: the row factors of the
    // chunk's first 4 * kThreads rows for the weight pre-scale, issued with
    // the first prefetch so that both arrive in one memory latency (rows past
    // the chunk read 0)
    float f_early[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (!GATHER) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            f_early[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       cbuf.scales, (tid + u * kThreads) * 4, 0, 0));
    }

    // append variant: the workgroups whose chunk holds the new row encode it
    // themselves, and its codes and scale replace whatever the loads above
    // and below read of that row (the LDS tile row, the row factors, the
    // pre-scale maximum); one of them writes it to the cache.  Every wave
    // loads the whole f32 row (lane l: dims 4l .. 4l+3 and 256 + 4l .. +3).
    // (the loads go through a buffer range that is empty in the other
    // workgroups: no branch, so no wait for the loads already in flight)
    bool has_new = false;
    int new_rel = 0;
    f32x4 xn0 = {0.0f, 0.0f, 0.0f, 0.0f}, xn1 = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (APPEND) {
        has_new = a.new_row >= c0 && a.new_row < c1;
        new_rel = (int)(a.new_row - c0);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.x_new), (short)0, has_new ? D * 4 : 0, kBufWord3);
        xn0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * lane, 0, 0));
        xn1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, 4 * HALF + 16 * lane, 0, 0));
    }

    if constexpr (FMT == KVQ_TQ4) {
        // byte -> (f16 level of the low nibble, f16 level of the high nibble)
        // (the 16 levels are read as uniform values and selected per lane: a
        // per-lane load here would wait behind the prefetch issued above)
        if (tid < 256) {
            const int nlo = tid & 15, nhi = tid >> 4;
            float llo = a.level[0], lhi = a.level[0];
#pragma unroll
            for (int k = 1; k < 16; ++k) {
                llo = nlo == k ? a.level[k] : llo;
                lhi = nhi == k ? a.level[k] : lhi;
            }
            lut_s[tid] = f16_bits_rne(llo) | (f16_bits_rne(lhi) << 16);
        }
    }

    // ---- query: q * 2^eq as f16 high + f16 residual, staged in LDS ----
    // thread t: head t/32, dims 16*(t%32) .. +16; the 32 threads of a head sit
    // in one half-wave, so cross-thread steps are butterflies over 5 lane bits
    __shared__ float qs_s[16];
    // the workgroup's query rows through a buffer range that ends at its last
    // head: a missing head reads zeros, and the loads need no branch (a
    // branch here made the compiler wait for the prefetch above before the
    // remaining query loads)
    const __amdgpu_buffer_rsrc_t qbuf = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.q + qrow0 * QW), (short)0, hv * QW * 4, kBufWord3);
    {
        const int head = tid >> 5, part = tid & 31;
        const int qoff = (head * QW + 16 * part) * 4;
        float x[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x4 u = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qbuf, qoff + 16 * k, 0, 0));
            x[4 * k] = u[0]; x[4 * k + 1] = u[1]; x[4 * k + 2] = u[2]; x[4 * k + 3] = u[3];
        }
        if constexpr (FMT == KVQ_TQ4) {
            // q' = H D q: sign flips of the encoder's rotation, then the
            // unnormalised Walsh-Hadamard transform (strides 1..8 inside the
            // thread, 16..256 across the head's 32 threads)
            const uint64_t w = splitmix64_at(a.seed, (uint64_t)(part >> 2));
            const int sh = (16 * part) & 63;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if ((w >> (sh + e)) & 1ull) x[e] = -x[e];
#pragma unroll
            for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (i & h) continue;
                    const float u = x[i], v = x[i + h];
                    x[i] = u + v;
                    x[i + h] = u - v;
                }
            }
            auto stage = [&](auto xl, int m) {
                const bool upper = (part >> m) & 1;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float y = xl(x[e]);
                    x[e] = upper ? (y - x[e]) : (x[e] + y);
                }
            };
            stage([](float v) { return xor_lane<1>(v); }, 0);
            stage([](float v) { return xor_lane<2>(v); }, 1);
            stage([](float v) { return xor_lane<4>(v); }, 2);
            stage([](float v) { return xor_lane<8>(v); }, 3);
            stage([](float v) { return xor_lane<16>(v); }, 4);
        }
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(x[e]));
        mx = fmaxf(mx, xor_lane<16>(mx));
        mx = fmaxf(mx, xor_lane<8>(mx));
        mx = fmaxf(mx, xor_lane<4>(mx));
        mx = fmaxf(mx, xor_lane<2>(mx));
        mx = fmaxf(mx, xor_lane<1>(mx));
        const int eq = headroom_exp(mx);
        half8_t hi[2], lo[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float xs = ldexpf(x[e], eq);
            const _Float16 hh = (_Float16)xs;
            hi[e >> 3][e & 7] = hh;
            lo[e >> 3][e & 7] = (_Float16)(xs - (float)hh);
        }
        uint8_t* dst = lds + q_stage_off<FMT>() + head * QROW * 2 + 32 * part;
        *reinterpret_cast<half8_t*>(dst) = hi[0];
        *reinterpret_cast<half8_t*>(dst + 16) = hi[1];
        *reinterpret_cast<half8_t*>(dst + QROW) = lo[0];
        *reinterpret_cast<half8_t*>(dst + QROW + 16) = lo[1];
        if (part == 0) qs_s[head] = ldexpf(1.0f, -eq - F::LOG2_ROW_DIV) * a.sm_scale * kLog2e;
    }

    if constexpr (ROPE) {
        // rope query part: thread t < 256 takes head t/16, dims 4*(t%16) .. +4
        // (TQ4: q'_rope = H D q_rope with the rope seed, strides 1, 2 inside
        // the thread and 4 .. 32 across the head's 16 threads), then
        // * 2^eq_rope as f16 high + residual
        if (tid < 256) {
            const int head = tid >> 4, part = tid & 15;
            const f32x4 u = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                          qbuf, (head * QW + D + 4 * part) * 4, 0, 0));
            float x[4] = {u[0], u[1], u[2], u[3]};
            if constexpr (FMT == KVQ_TQ4) {
                const uint64_t w = splitmix64_at(a.rseed, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((w >> (4 * part + e)) & 1ull) x[e] = -x[e];
#pragma unroll
                for (int h = 1; h < 4; h <<= 1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (i & h) continue;
                        const float p0 = x[i], p1 = x[i + h];
                        x[i] = p0 + p1;
                        x[i + h] = p0 - p1;
                    }
                }
                auto stage = [&](auto xl, int m) {
                    const bool upper = (part >> m) & 1;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float y = xl(x[e]);
                        x[e] = upper ? (y - x[e]) : (x[e] + y);
                    }
                };
                stage([](float v) { return xor_lane<1>(v); }, 0);
                stage([](float v) { return xor_lane<2>(v); }, 1);
                stage([](float v) { return xor_lane<4>(v); }, 2);
                stage([](float v) { return xor_lane<8>(v); }, 3);
            }
            float mx = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
            mx = fmaxf(mx, xor_lane<8>(mx));
            mx = fmaxf(mx, xor_lane<4>(mx));
            mx = fmaxf(mx, xor_lane<2>(mx));
            mx = fmaxf(mx, xor_lane<1>(mx));
            const int eqr = headroom_exp(mx);
            _Float16* dst = qr_s + head * 2 * DR + 4 * part;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float xs = ldexpf(x[e], eqr);
                const _Float16 hh = (_Float16)xs;
                dst[e] = hh;
                dst[DR + e] = (_Float16)(xs - (float)hh);
            }
            if (part == 0)
                qrs_s[head] = ldexpf(1.0f, -eqr - (FMT == KVQ_TQ4 ? 6 : 0)) * a.sm_scale * kLog2e;
        }
    }

    // ---- append variant: the new row's scale and this lane's codes ----
    // (the KV8 encoder's arithmetic: s = fl(amax / 448), codes e4m3(x / s),
    // a zero row stores scale 0 and zero codes)
    float new_s = 0.0f;
    uint32_t new_w = 0;                             // dims 256 half + 4 lane .. +3
    if constexpr (APPEND) {
        if (has_new) {
            const float m = fmaxf(fmaxf(fmaxf(fabsf(xn0[0]), fabsf(xn0[1])), fmaxf(fabsf(xn0[2]), fabsf(xn0[3]))),
                                  fmaxf(fmaxf(fabsf(xn1[0]), fabsf(xn1[1])), fmaxf(fabsf(xn1[2]), fabsf(xn1[3]))));
            const float s = wave_max(m) / 448.0f;
            const bool live = s > 0.0f;
            new_s = live ? s : 0.0f;
            uint32_t w0 = 0, w1 = 0;
            if (live) {
                w0 = e4m3x4(xn0[0] / s, xn0[1] / s, xn0[2] / s, xn0[3] / s);
                w1 = e4m3x4(xn1[0] / s, xn1[1] / s, xn1[2] / s, xn1[3] / s);
            }
            new_w = half ? w1 : w0;
            if (hg == 0 && wave == 0) {
                *reinterpret_cast<uint32_t*>(a.new_codes + 4 * lane) = w0;
                *reinterpret_cast<uint32_t*>(a.new_codes + HALF + 4 * lane) = w1;
                if (lane == 0) *a.new_scale = new_s;
            }
        }
    }

    // ---- weight pre-scale: max row factor of the chunk ----
    float smax = 0.0f;
    if (n_tiles <= kPairs) {
        // one tile per pair: the first prefetch already holds every row factor
        // of the chunk (rows past the chunk count 0; no second pass over HBM)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r = pair * TR + rho(g, e);
            float f = row_factor<GATHER>(pf, g, e);
            if (APPEND && has_new && r == new_rel) f = new_s;
            if (r < n_rows32) smax = fmaxf(smax, f);
        }
    }
    if (!GATHER && n_tiles > kPairs) {
        if constexpr (APPEND) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (has_new && tid + u * kThreads == new_rel) f_early[u] = new_s;
        }
        smax = fmaxf(fmaxf(f_early[0], f_early[1]), fmaxf(f_early[2], f_early[3]));
    }
    // (dense: the rows after the first 4 * kThreads; gather: every listed row)
    const int64_t t_first = GATHER ? c0 + tid : c0 + tid + 4 * kThreads;
    for (int64_t t0 = t_first; n_tiles > kPairs && t0 < c1; t0 += 4 * kThreads) {   // 4 loads in flight per round
        float f[4];
        if (idx == nullptr) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t t = t0 + u * kThreads;
                f[u] = t < c1 ? a.scales[t] : 0.0f;
                if (APPEND && has_new && t == a.new_row) f[u] = new_s;
            }
        } else {
            // gather: list entries, then the listed rows' factors, all loads
            // unconditional (masked afterwards)
            int32_t ent[4];
            float sv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t t = t0 + u * kThreads;
                ent[u] = idx[t < c1 ? t : c1 - 1];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) sv[u] = a.scales[listed_row(ent[u], a.n_cache)];
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int64_t t = t0 + u * kThreads;
                f[u] = (t < c1 && ent[u] >= 0 && ent[u] < a.n_cache) ? sv[u] : 0.0f;
            }
        }
        smax = fmaxf(smax, fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])));
    }
    smax = wave_max(smax);
    if (lane == 0) red_s[wave] = smax;
    __syncthreads();
    const float qk_scale = qs_s[n16];
    const float qkr_scale = ROPE ? qrs_s[n16] : 0.0f;
    half8_t qhi[KSTEPS], qlo[KSTEPS];
    {
        const uint8_t* qrow = lds + q_stage_off<FMT>() + n16 * QROW * 2 + 2 * HALF * half;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            qhi[s] = *reinterpret_cast<const half8_t*>(qrow + 2 * q_dim<FMT>(s, g));
            qlo[s] = *reinterpret_cast<const half8_t*>(qrow + QROW + 2 * q_dim<FMT>(s, g));
        }
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) smax = fmaxf(smax, red_s[w]);
    const int ew = headroom_exp(smax) - kWeightShift;
    const float w_scale = ldexpf(1.0f, ew);
    if constexpr (q_stage_off<FMT>() == 0) __syncthreads();   // query staging area is reused below

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, m_used = -INFINITY, l_run = 0.0f;

    // per-lane LDS offsets (the loops below add immediates only)
    const uint8_t* pa = tile + n16 * LDR + 8 * g;                   // score tile 0 row n16
    const uint8_t* pb = pa + 16 * LDR;                              // score tile 1 row 16+n16
    // V operand sources: KV8 rows rho(g, n16/2) for ds_read_b64_tr_b8; TQ4 rows
    // 4g + n16/4 (and 16 more) for ds_read_b64_tr_b16
    const uint8_t* pv = (FMT == KVQ_FP8) ? tile + rho(g, n16 >> 1) * LDR + 8 * (n16 & 1)
                                         : tile + (4 * g + (n16 >> 2)) * LDR + 8 * (n16 & 3);

    for (int it = 0; it < n_iter; ++it) {
        const int j = pair + kPairs * it;
        const bool live_tile = j < n_tiles;
        const int rel0 = j * TR;                        // first row of the tile in the chunk
        const int64_t row0 = c0 + rel0;
        float srow[8], wrow[8];                         // score and weight row factors
        const PfRegs<FMT> cur = pf;
        const RopeRegs<FMT> rcur = rpf;
        if constexpr (FMT == KVQ_FP8) {
            uint8_t* pw = tile + (lane / F::LPR) * LDR + 16 * (lane % F::LPR);
#pragma unroll
            for (int k = 0; k < F::NLD; ++k) *reinterpret_cast<u32x4*>(pw + F::RPL * k * LDR) = cur.v[k];
        }
        if constexpr (!ROPE) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                srow[e] = row_factor<GATHER>(cur, g, e) * qk_scale;
                wrow[e] = row_factor<GATHER>(cur, g, e) * w_scale;
            }
        }   // (with a rope part both are formed where used: fewer live registers)
        if constexpr (APPEND) {
            if (has_new && j == new_rel / TR) {
                // the new row over what the load read of it (same wave: the
                // LDS writes land in order)
                *reinterpret_cast<uint32_t*>(tile + (new_rel % TR) * LDR + 4 * lane) = new_w;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (rel0 + rho(g, e) == new_rel) {
                        srow[e] = new_s * qk_scale;
                        wrow[e] = new_s * w_scale;
                    }
            }
        }
        if constexpr (GATHER)
            prefetch<FMT>(pf, a.codes, a.scales, row0 + (int64_t)kPairs * TR, a.T, half, lane, g, idx,
                          a.n_cache);
        else
            prefetch_dense<FMT>(pf, cbuf, rel0 + kPairs * TR, half, lane, g);

        // partial scores over this wave's half of the dims
        // four independent accumulation chains (high / residual query part x
        // two row tiles) keep the matrix pipe busy; summed once per tile
        f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 s0l = {0.0f, 0.0f, 0.0f, 0.0f}, s1l = {0.0f, 0.0f, 0.0f, 0.0f};
        if (live_tile) {
            if constexpr (FMT == KVQ_FP8) {
                uint2 ka[KSTEPS], kb[KSTEPS];
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    ka[s] = *reinterpret_cast<const uint2*>(pa + 32 * s);
                    kb[s] = *reinterpret_cast<const uint2*>(pb + 32 * s);
                }
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    const half8_t A0 = cvt8(ka[s].x, ka[s].y);
                    const half8_t A1 = cvt8(kb[s].x, kb[s].y);
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qhi[s], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qhi[s], s1, 0, 0, 0);
                    s0l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qlo[s], s0l, 0, 0, 0);
                    s1l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qlo[s], s1l, 0, 0, 0);
                }
            } else {
                // k-steps 2u, 2u+1: the 8 bytes at 32u + 8g of rows n16, 16+n16,
                // decoded here; the decoded rows also go to the f16 tile (dims
                // 64u + 16g + 8h at byte 2 * that) for the context
                uint8_t* w0 = tile + n16 * LDR + 32 * g;
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s) {
                    const int u = s >> 1;
                    const uint32_t xa = (s & 1) ? cur.v[0][u].y : cur.v[0][u].x;
                    const uint32_t xb = (s & 1) ? cur.v[1][u].y : cur.v[1][u].x;
                    const half8_t A0 = lut8(lut_s, xa);
                    const half8_t A1 = lut8(lut_s, xb);
                    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qhi[s], s0, 0, 0, 0);
                    s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qhi[s], s1, 0, 0, 0);
                    s0l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qlo[s], s0l, 0, 0, 0);
                    s1l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qlo[s], s1l, 0, 0, 0);
                    *reinterpret_cast<half8_t*>(w0 + 128 * u + 16 * (s & 1)) = A0;
                    *reinterpret_cast<half8_t*>(w0 + 16 * LDR + 128 * u + 16 * (s & 1)) = A1;
                }
            }
        }
        s0 += s0l;
        s1 += s1l;
        if constexpr (ROPE) {
            // rope k-step: this wave's 32 rope dims of both row tiles
            f32x4 r0 = {0.0f, 0.0f, 0.0f, 0.0f}, r1 = {0.0f, 0.0f, 0.0f, 0.0f};
            if (live_tile) {
                const _Float16* qr = qr_s + n16 * 2 * DR + 32 * half + 8 * g;
                const half8_t qrh = *reinterpret_cast<const half8_t*>(qr);
                const half8_t qrl = *reinterpret_cast<const half8_t*>(qr + DR);
                half8_t R0, R1;
                if constexpr (FMT == KVQ_FP8) {
                    R0 = cvt8(rcur.v[0].x, rcur.v[0].y);
                    R1 = cvt8(rcur.v[1].x, rcur.v[1].y);
                } else {
                    R0 = lut8(lut_s, rcur.v[0]);
                    R1 = lut8(lut_s, rcur.v[1]);
                }
                r0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(R0, qrh, r0, 0, 0, 0);
                r1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(R1, qrh, r1, 0, 0, 0);
                r0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(R0, qrl, r0, 0, 0, 0);
                r1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(R1, qrl, r1, 0, 0, 0);
            }
            // the two key parts have their own row factors: scale before the
            // exchange (the sums below are then the finished scores)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s0[i] = s0[i] * (row_factor<GATHER>(cur, g, i) * qk_scale) +
                        r0[i] * (rope_factor<GATHER>(rcur, g, i) * qkr_scale);
                s1[i] = s1[i] * (row_factor<GATHER>(cur, g, 4 + i) * qk_scale) +
                        r1[i] * (rope_factor<GATHER>(rcur, g, 4 + i) * qkr_scale);
            }
            // next tile's rope operands (issued once this tile's are consumed)
            if constexpr (GATHER)
                prefetch_rope<FMT>(rpf, a.rcodes, a.rscales, row0 + (int64_t)kPairs * TR, a.T, half, n16,
                                   g, idx, a.n_cache);
            else
                prefetch_rope_dense<FMT>(rpf, rbuf, rel0 + kPairs * TR, half, n16, g);
        }
        // add the partner's half (identical sums in both waves: a + b == b + a)
        const int buf = (F::EXCH_BUFS == 2) ? (it & 1) : 0;
        float* mine = exch + (buf * kWaves + wave) * 512 + lane * 8;
        const float* other = exch + (buf * kWaves + (wave ^ 1)) * 512 + lane * 8;
        *reinterpret_cast<f32x4*>(mine) = s0;
        *reinterpret_cast<f32x4*>(mine + 4) = s1;
        __syncthreads();
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(other);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(other + 4);
        if constexpr (F::EXCH_BUFS == 1) __syncthreads();   // exchange read before it is rewritten
        if (!live_tile) continue;
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (ROPE) {
                sc[i] = s0[i] + o0[i];
                sc[4 + i] = s1[i] + o1[i];
            } else {
                sc[i] = (s0[i] + o0[i]) * srow[i];
                sc[4 + i] = (s1[i] + o1[i]) * srow[4 + i];
            }
        }
        if (rel0 + TR > n_rows32) {                     // ragged tile: mask rows past the chunk
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (rel0 + rho(g, e) >= n_rows32) sc[e] = -INFINITY;
        }
        if constexpr (GATHER) {                         // skip padding entries (factor -0.0)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (__builtin_signbit(row_factor<GATHER>(cur, g, e))) sc[e] = -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = fmaxf(tmax, xor_lane<16>(tmax));
        tmax = fmaxf(tmax, xor_lane<32>(tmax));
        if (tmax == -INFINITY) continue;                // gather: only padding entries in this tile
        m_run = fmaxf(m_run, tmax);
        const bool need = m_run > m_used + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
            // nothing accumulated yet while every head's max is still -inf
            const bool started = __builtin_amdgcn_ballot_w64(m_used != -INFINITY) != 0ull;
            const float m_new = need ? m_run : m_used;
            const float alpha = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - m_new);
            l_run *= alpha;
            m_used = m_new;
            if (started) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[t][i] *= ai;
                }
            }
        }
        half8_t phi, plo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(sc[e] - m_used);
            l_run += p;
            // the f32 product is rounded, then split (opaque: no fused
            // multiply-convert, so every variant rounds the same way)
            const float w = opaque(p * (ROPE ? row_factor<GATHER>(cur, g, e) * w_scale : wrow[e]));
            const _Float16 h = (_Float16)w;
            phi[e] = h;
            plo[e] = (_Float16)(w - (float)h);
        }

        // context over this wave's 256 dims: V operand by transpose read
        if constexpr (FMT == KVQ_FP8) {
            // (the rope variant reads the V operands in two rounds: fewer live registers)
            constexpr int VCH = ROPE ? NT / 2 : NT;
#pragma unroll
            for (int t0 = 0; t0 < NT; t0 += VCH) {
                i32x2 vv[VCH];
#pragma unroll
                for (int t = 0; t < VCH; ++t)
                    vv[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (i32x2 __attribute__((address_space(3)))*)(pv + 16 * (t0 + t)));
#pragma unroll
                for (int t = 0; t < VCH; ++t) {
                    const half8_t B = cvt8((uint32_t)vv[t].x, (uint32_t)vv[t].y);
                    acc[t0 + t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi, B, acc[t0 + t], 0, 0, 0);
                    acc[t0 + t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo, B, acc[t0 + t], 0, 0, 0);
                }
            }
        } else {
            // decoded f16 rows: rows rho(g, 0..3) and rho(g, 4..7), column 16t + n16
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(pv + 32 * t));
                const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(pv + 16 * LDR + 32 * t));
                const half8_t B = __builtin_shufflevector(__builtin_bit_cast(half4_t, h0),
                                                          __builtin_bit_cast(half4_t, h1),
                                                          0, 1, 2, 3, 4, 5, 6, 7);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(phi, B, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(plo, B, acc[t], 0, 0, 0);
            }
        }
    }

    // ---- merge the 4 pairs in LDS, write the chunk partial ----
    l_run += xor_lane<16>(l_run);
    l_run += xor_lane<32>(l_run);
    __syncthreads();                                    // tiles and exchange consumed
    if (half == 0 && g == 0) {
        ml_s[pair][n16][0] = m_used;
        ml_s[pair][n16][1] = l_run;
    }
    // unscaled accumulators; the reader applies each pair's factor
    float* red = reinterpret_cast<float*>(lds);        // [4 pairs][16 heads][MROW]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float* dst = red + (pair * 16 + 4 * g + i) * MROW + HALF * half;
#pragma unroll
        for (int t = 0; t < NT; ++t) dst[16 * t + n16] = acc[t][i];   // tile t: dims 16t + n16
    }
    __syncthreads();
    // head h: M = max of the pairs' running maxima, pair factors 2^(m_p - M), L
    auto head_ml = [&](int h, float* f, float& M, float& L) {
        M = -INFINITY;
#pragma unroll
        for (int p = 0; p < kPairs; ++p) M = fmaxf(M, ml_s[p][h][0]);
        L = 0.0f;
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            const float mp = ml_s[p][h][0];
            f[p] = (mp == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mp - M);
            L += f[p] * ml_s[p][h][1];
        }
    };
    if (tid < hv) {
        float f[kPairs], M, L;
        head_ml(tid, f, M, L);
        if (a.direct) {
            if (a.lse != nullptr) a.lse[qrow0 + tid] = (M + log2f(L)) * 0.69314718055994531f;
        } else {
            float* ml = a.part_ml + ((int64_t)chunk * n_qrows + qrow0 + tid) * 2;
            ml[0] = M;
            ml[1] = L;
        }
    }
    const float unscale = ldexpf(1.0f, -ew - F::LOG2_ROW_DIV);
    auto merged = [&](int idx, float& L) {
        const int h = idx / (D / 4), dd = 4 * (idx % (D / 4));
        float f[kPairs], M;
        head_ml(h, f, M, L);
        f32x4 s = *reinterpret_cast<const f32x4*>(red + h * MROW + dd) * f[0];
#pragma unroll
        for (int p = 1; p < kPairs; ++p) s += *reinterpret_cast<const f32x4*>(red + (p * 16 + h) * MROW + dd) * f[p];
        return s * unscale;
    };
    if (a.direct) {
        for (int idx = tid; idx < hv * D / 4; idx += kThreads) {
            const int h = idx / (D / 4), dd = 4 * (idx % (D / 4));
            float L;
            const f32x4 m = merged(idx, L);
            // no listed row at all (gather with only padding): out = 0, lse = -inf
            const f32x4 v = L > 0.0f ? m / L : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            *reinterpret_cast<f32x4*>(a.out + (qrow0 + h) * D + dd) = v;
        }
    } else {
        // read once, by the combine pass: streaming stores
        float* dst = a.part_acc + ((int64_t)chunk * n_qrows + qrow0) * D;
        for (int idx = tid; idx < hv * D / 4; idx += kThreads) {
            float L;
            __builtin_nontemporal_store(merged(idx, L), reinterpret_cast<f32x4*>(dst + 4 * idx));
        }
    }
}

template <int FMT, bool ROPE, bool GATHER, bool APPEND = false>
hipError_t launch_variant(const MlaArgs& a, int blocks, hipStream_t s) {
    constexpr int lds = dyn_lds<FMT>();
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_dyn_lds_once(reinterpret_cast<const void*>(&k_mla_mfma<FMT, ROPE, GATHER, APPEND>),
                                    lds, lds_set);
    if (e != hipSuccess) return e;
    k_mla_mfma<FMT, ROPE, GATHER, APPEND><<<blocks, kThreads, lds, s>>>(a);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const MlaArgs& a, bool rope, int blocks, hipStream_t s) {
    if (a.idx != nullptr)
        return rope ? launch_variant<FMT, true, true>(a, blocks, s)
                    : launch_variant<FMT, false, true>(a, blocks, s);
    return rope ? launch_variant<FMT, true, false>(a, blocks, s)
                : launch_variant<FMT, false, false>(a, blocks, s);
}

}  // namespace

bool mla_mfma_eligible(const kvq_cache& kv, int32_t Hq, int32_t S, const void* q) {
    // 16-byte vector loads of codes, row factors and the query
    const bool al = (reinterpret_cast<uintptr_t>(kv.codes) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(kv.scales) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(q) % 16 == 0);
    const int64_t blocks = (int64_t)(Hq + 15) / 16 * S;     // per chunk
    // rope part: 64 wide, rows and row factors 16-byte aligned
    const bool rope_ok = kv.d_rope == 0 ||
                         (kv.d_rope == DR && reinterpret_cast<uintptr_t>(kv.rope_codes) % 16 == 0 &&
                          reinterpret_cast<uintptr_t>(kv.rope_scales) % 16 == 0);
    return (kv.fmt == KVQ_FP8 || kv.fmt == KVQ_TQ4) && kv.d == D && rope_ok && Hq >= 1 &&
           kv.n_kv == 1 && al && blocks <= (1 << 22);
}

// workspace: partials, n_split x (S * Hq) x (D + 2) floats.  Decode splits T
// into ~256 / (Hq/16) chunks (about one workgroup per CU); a prefill with many
// tokens already has enough workgroups and keeps one chunk per token.
void mla_mfma_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p, bool wide_decode) {
    if (mla_prefill_kv8_eligible(kv, Hq, S)) {
        mla_prefill_kv8_plan(kv, Hq, S, p);
        return;
    }
    if (wide_decode && mla_decode64_eligible(kv, Hq, S)) {
        mla_decode64_plan(kv, Hq, S, p);
        return;
    }
    const int64_t n_hg = (Hq + 15) / 16;
    const int64_t T = kv.n_rows;
    int64_t want = (256 + n_hg * S - 1) / (n_hg * S);
    if (want < 1) want = 1;
    int64_t chunk = (T + want - 1) / want;
    chunk = ((chunk + 127) / 128) * 128;                    // whole 32-row tiles for 4 pairs
    // chunk bytes (and the prefetch one round past them) stay within the
    // 32-bit offsets of the kernel's buffer loads
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    p.chunk = chunk;
    p.n_split = (int32_t)((T + chunk - 1) / chunk);
    p.n_qrows = Hq * S;
    p.heads_per_blk = 16;
    p.n_qgroups = (int32_t)(n_hg * S);
    p.log2_domain = 1;
    p.ws_bytes = (size_t)p.n_split * p.n_qrows * (D + 2) * sizeof(float);
}

hipError_t launch_mla_mfma(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                           int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                           float* part_ml, float* out, float* lse, hipStream_t s,
                           const int32_t* idx, int64_t n_cache, const NewRow* nr) {
    if (nr != nullptr && !mla_append_fusable(kv, p, Hq, S, pos0, idx, nr)) return hipErrorInvalidValue;
    if (idx == nullptr && mla_prefill_kv8_eligible(kv, Hq, S))
        return launch_mla_prefill_kv8(kv, p, q, Hq, S, pos0, sm_scale, part_acc, part_ml, out, lse, s);
    if (idx == nullptr && pos0 < 0 && p.heads_per_blk == 64 && mla_decode64_eligible(kv, Hq, S))
        return launch_mla_decode64(kv, p, q, Hq, S, pos0, sm_scale, part_acc, part_ml, out, lse, s);
    if (idx != nullptr && (S != 1 || pos0 >= 0)) return hipErrorInvalidValue;
    MlaArgs a;
    a.idx = idx;
    a.n_cache = idx != nullptr ? n_cache : kv.n_rows;
    a.direct = (p.n_split == 1) ? 1 : 0;
    a.out = out;
    a.lse = lse;
    a.codes = kv.codes;
    a.scales = reinterpret_cast<const float*>(kv.scales);
    a.q = q;
    a.sm_scale = sm_scale;
    a.T = kv.n_rows;
    a.Hq = Hq;
    a.S = S;
    a.pos0 = pos0;
    a.chunk = p.chunk;
    const int blocks = p.n_split * ((Hq + 15) / 16) * S;
    a.xcd_map = (blocks % 8 == 0) ? 1 : 0;
    a.part_acc = part_acc;
    a.part_ml = part_ml;
    a.seed = kv.rot_seed;
    a.rcodes = kv.rope_codes;
    a.rscales = kv.rope_scales;
    a.rseed = kv.rope_seed;
    const Codebook16& cb = codebook16();
    for (int i = 0; i < 16; ++i) a.level[i] = cb.level[i];
    a.x_new = nullptr;
    a.new_codes = nullptr;
    a.new_scale = nullptr;
    a.new_row = -1;
    if (nr != nullptr) {
        a.x_new = nr->x;
        a.new_codes = nr->codes + nr->row * D;
        a.new_scale = nr->scales + nr->row;
        a.new_row = nr->row;
        return launch_variant<KVQ_FP8, false, false, true>(a, blocks, s);
    }
    const bool rope = kv.d_rope != 0;
    if (kv.fmt == KVQ_TQ4)
        return launch_fmt<KVQ_TQ4>(a, rope, blocks, s);
    return launch_fmt<KVQ_FP8>(a, rope, blocks, s);
}

// The per-head-group KV8 decode of one token over the whole cache, dense rows
// without a rope part, with the new row inside the cache and 16-byte aligned.
bool mla_append_fusable(const kvq_cache& kv, const AttnPlan& p, int32_t Hq, int32_t S, int64_t pos0,
                        const int32_t* idx, const NewRow* nr) {
    return nr != nullptr && p.path == 1 && p.heads_per_blk == 16 && kv.fmt == KVQ_FP8 && kv.d == D &&
           kv.d_rope == 0 && idx == nullptr && S == 1 && pos0 < 0 && mla_mfma_eligible(kv, Hq, S, nr->x) &&
           !mla_prefill_kv8_eligible(kv, Hq, S) && nr->row >= 0 && nr->row < kv.n_rows &&
           nr->codes == kv.codes && nr->scales == reinterpret_cast<const float*>(kv.scales);
}

}  // namespace kvq
