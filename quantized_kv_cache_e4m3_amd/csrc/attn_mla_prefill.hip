// Shared-tile flash attention for the MLA latent (d = 512, heads in groups
// of 16) on the gfx950 matrix cores: the KV8 chunked prefill (4 tokens x 16
// heads per workgroup) and the TQ4 decode of 64 heads (1 token x 4 head
// groups per workgroup).
//
// [colibri #553] "What's in it" / [colibri #399] "Commits" item 2: the rows
// are consumed as they are stored and the latent row is both key and value.
// KV8: fp8 e4m3 values, the f32 row scale outside the dot product; token s of
// a prefill attends rows t <= pos0 + s.  TQ4 ([colibri #553] "What's in it",
// "Ready for review" comment): 4-bit codebook indices with the row radius
// outside the dot product; the query is rotated once per head (q' = H D q),
// the scores are (r/n) q'.c with c the codebook values, the context stays in
// the rotated domain and is unrotated once by the combine step.
//
// Both products run on v_mfma_f32_16x16x32_f16 with exact f16 operands: e4m3
// values and the fp16-rounded codebook levels are exact in f16, and the f32
// side (query, weights p * row factor) is split into an f16 high part and an
// f16 residual multiplied in two passes, pre-scaled by powers of two.
//
// Work layout.  A workgroup has 4 waves, one per SIMD, and 4 units of 16
// query rows: the prefill's units are 4 consecutive tokens of one head group,
// the decode's the 4 head groups of its token.  Wave w scores unit w over the
// full width (query operands for 512 dims in 128 registers) and runs that
// unit's online softmax, so no partial scores are exchanged and no softmax is
// computed twice.  The context is split by dims: waves 2p and 2p + 1 both
// accumulate units 2p and 2p + 1, wave 2p + h on dims [256h, 256h + 256) (128
// accumulator registers), reading the partner's weights from LDS, so each
// context operand read feeds two units.  Each 32-row tile is loaded once
// (prefetched into registers; a wave loads and later stores 8 whole rows),
// converted once to f16 by the workgroup (KV8: hardware fp8 conversion; TQ4:
// a 256-entry LDS table maps one packed byte to the f16 levels of its two
// nibbles) into one of four LDS tile buffers (1040-byte rows, with the tile's
// row factors behind them), and read by all waves: score operands as 16-byte
// row reads, context operands by ds_read_b64_tr_b16 (8 rows of one dim per
// lane, in the order rho(g, e) in which the score accumulators hold the
// weights).  So a decode converts each row once for its 64 heads.
//
// The tile loop is software-pipelined with one barrier per tile: iteration j
// runs the softmax of tile j beside the scores of tile j + 1 and publishes the
// weights of tile j, and the context of tile j - 1 (both units' weights
// published the iteration before) beside the conversion of tile j + 2 and the
// loads of tile j + 3.  A raised reference maximum rescales the accumulators
// in a rarely taken branch through an LDS round trip, so the accumulators are
// only ever touched by the matrix cores.  Tiles that reach past a unit's row
// limit (a prefill token's causal limit, the chunk's end) run a second copy of
// the loop with the row mask.  With one chunk each wave writes the normalized
// output of its pair's two units on its dims and the lse of its unit;
// otherwise the rows are split into chunks and the same places get
// (m, l, acc) partials for the combine step.
#include <math.h>

#include <type_traits>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 512;
constexpr int HALF = D / 2;
constexpr int TR = 32;                  // rows per tile
constexpr int KSTEPS = D / 32;          // 16 score k-steps (full width)
constexpr int NT = HALF / 16;           // 16 context dim tiles per wave
constexpr int kWaves = 4;               // one per SIMD
constexpr int kTok = 4;                 // tokens per workgroup, one scored per wave
constexpr int kThreads = 64 * kWaves;
constexpr int LDR = 2 * D + 16;         // f16 tile row stride (bytes)
constexpr int TILE_F16 = TR * LDR;
constexpr int TILE_BYTES = TILE_F16 + TR * 4;       // + the tile's row scales
constexpr int kBufs = 4;
// a wave's published tile: weights hi [lane] 16 B, lo [lane] 16 B and the
// per-head rescale factors (the flags sit in a small array of their own)
constexpr int EX_LO = 64 * 16, EX_ALPHA = 2 * 64 * 16;
constexpr int EXCH_WAVE = EX_ALPHA + 16 * 4;
constexpr int EXCH_BYTES = 2 * kWaves * EXCH_WAVE;  // double-buffered
constexpr int SCR_WAVE = 2 * 64 * 16;               // rescale round trip: 2 f32x4 per lane
constexpr int SCR_OFF = kBufs * TILE_BYTES + EXCH_BYTES;
constexpr int kLoopLds = SCR_OFF + kWaves * SCR_WAVE;
constexpr int OUT_ROW = HALF + 4;       // output staging row (floats)
constexpr int kOutLds = kWaves * 2 * 16 * OUT_ROW * 4;
constexpr int kDynLds = kLoopLds > kOutLds ? kLoopLds : kOutLds;
static_assert(kDynLds <= 160 * 1024 - 1024, "LDS budget");
static_assert(TILE_BYTES % 16 == 0 && EXCH_WAVE % 16 == 0, "16-byte aligned LDS buffers");
static_assert(NT / 2 == TR / kWaves, "one converted row of a wave per pair of context dim tiles");
constexpr float kRescaleSlack = 8.0f;   // log2 units: p <= 2^8 between rescales
constexpr int kWeightShift = 7;         // 2^ew * (max row scale) in [2^6, 2^7): weights < 2^15
constexpr float kLog2e = 1.4426950408889634f;
// TQ4 decode with all heads per workgroup from this many rows: below it the
// per-head-group kernel is faster (measured, 64 heads: 26.5 against 42.2 us at
// 16384 rows, 49.5 against 49.7 at 73728, 52.8 against 50.8 at 81920, 71.2
// against 62.0 at 131072), as the all-heads path's fixed costs (query
// preparation, 256 chunk partials) outweigh its single decode per row
constexpr int64_t kDecode64MinRows = 77824;
// KV8 likewise, where the per-head-group kernel's cheaper rows (the fp8
// convert, no byte table) move the crossover further out (measured: 67.4
// against 68.5 us at 163840 rows, 74.6-76.7 against 72.8-72.9 at 196608, 88.6-89.3
// against 83.5-83.8 at 262144; 52.4 against 55.2 at 131072)
constexpr int64_t kDecode64MinRowsKv8 = 196608;

constexpr int kPrefill = 0, kDecode = 1;   // workgroup units: tokens of one head group / head groups of one token

// Per-format tile loads: a row's bytes and the 32-bit words per lane of a row
// (lane l holds dims 8l .. 8l + 7), and the power of two the row factor
// carries besides the score scale (TQ4: r / n with n = 512)
template <int FMT> struct TileFmt;
template <> struct TileFmt<KVQ_FP8> {
    static constexpr int ROWB = D, W = 2, LOG2_ROW_DIV = 0;
};
template <> struct TileFmt<KVQ_TQ4> {
    static constexpr int ROWB = D / 2, W = 1, LOG2_ROW_DIV = 9;
};

struct TileArgs {
    const uint8_t* codes;   // [T][row bytes]: e4m3 values, or packed nibbles (low first)
    const float* scales;    // [T]: row scale, or radius
    const float* q;         // [S][Hq][D]
    float sm_scale;
    int64_t T;
    int32_t Hq;
    int32_t S;
    int64_t pos0;
    int32_t xcd_map;
    int64_t chunk;          // rows per chunk (multiple of 32)
    int32_t n_split;        // chunks; 1: write out / lse directly
    float* part_acc;        // [n_split][S*Hq][D]
    float* part_ml;         // [n_split][S*Hq][2] (m in log2 units)
    float* out;             // [S][Hq][D]
    float* lse;             // [S][Hq] or null
    float level[16];        // TQ4 codebook (fp16 values)
    const _Float16* qhl;    // decode: prepared query, [Hq][high, residual][D] (else null)
    const float* qks;       // decode: its per-head score factors
};

__device__ __forceinline__ int headroom_exp(float x) {
    if (!(x > 0.0f)) return 0;
    int k;
    (void)frexpf(x, &k);
    return 14 - k;
}

// row of the tile held in context slot e of lane group g
__device__ __forceinline__ int rho(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

// The chunk's rows are read through buffer resources whose base is the
// chunk's first row and whose range ends at the last row the token group
// sees: a row past it reads as zeros without a memory access (such rows are
// masked by the causal limit), so offsets are 32-bit rows inside the chunk
// (the plan caps the chunk) and nothing is clamped per row.  The pipeline
// therefore loads, converts and scores the tiles past the last one without a
// branch.
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 (32-bit data format)
constexpr int64_t kMaxChunk = int64_t{1} << 21;
struct ChunkBufs {
    __amdgpu_buffer_rsrc_t codes, scales;
};

// wave w, lane l: the row bytes of dims 8l .. 8l + 7 of tile rows 8w + k
// (k < 8), and the factor of row (4w + l) % 32: a wave loads and stores whole
// rows, lane l the l-th 16 bytes of the f16 row, so the LDS stores are free
// of bank conflicts
template <int FMT>
struct TileRegs {
    uint32_t v[8][TileFmt<FMT>::W];
    float s;
};

template <int FMT>
__device__ __forceinline__ void load_tile(TileRegs<FMT>& r, const ChunkBufs& b, int rel0, int tid) {
    constexpr int ROWB = TileFmt<FMT>::ROWB, W = TileFmt<FMT>::W;
    const int w = tid >> 6, l = tid & 63;
    const int off = (rel0 + 8 * w) * ROWB + 4 * W * l;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int c = 0; c < W; ++c)      // (KV8: two 32-bit loads, merged into one 64-bit load)
            r.v[k][c] = __builtin_amdgcn_raw_buffer_load_b32(b.codes, off + k * ROWB + 4 * c, 0, 0);
    r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(b.scales, (rel0 + (tid & 31)) * 4, 0, 0));
}

// one prefetched row word set as the 8 f16 values of dims 8l .. 8l + 7
template <int FMT>
__device__ __forceinline__ u32x4 row_f16(const uint32_t (&v)[TileFmt<FMT>::W], const uint32_t* lut) {
    u32x4 h;
    if constexpr (FMT == KVQ_FP8) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const half2_t lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[c], 1.0f, false);
            const half2_t hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[c], 1.0f, true);
            h[2 * c] = __builtin_bit_cast(uint32_t, lo2);
            h[2 * c + 1] = __builtin_bit_cast(uint32_t, hi2);
        }
    } else {
        // byte i holds dims 8l + 2i (low nibble) and 8l + 2i + 1: one table word
#pragma unroll
        for (int i = 0; i < 4; ++i) h[i] = lut[(v[0] >> (8 * i)) & 0xFFu];
    }
    return h;
}

// the prefetched tile as f16 rows and its row factors (pipeline fill)
template <int FMT>
__device__ __forceinline__ void store_tile(uint8_t* buf, const TileRegs<FMT>& r, int tid, const uint32_t* lut) {
    const int w = tid >> 6, l = tid & 63;
    uint8_t* dst = buf + 8 * w * LDR + 16 * l;
#pragma unroll
    for (int k = 0; k < 8; ++k) *reinterpret_cast<u32x4*>(dst + k * LDR) = row_f16<FMT>(r.v[k], lut);
    // threads t and t + 32k hold the same row's factor: same-value stores, no branch
    reinterpret_cast<float*>(buf + TILE_F16)[tid & (TR - 1)] = r.s;
}

// scores of one tile for the wave's token over the full width: s[r] holds
// rows 16r + 4g + i (i = 0..3) of head n16.  The high query pass runs as two
// chains (even and odd k-steps), the residual pass as a third: scores reach
// hundreds in log2 units, where each float32 rounding of a long chain moves a
// weight, and two half-length chains halve the rounding error of the sum.
__device__ __forceinline__ void tile_scores(f32x4 (&sn)[2], const uint8_t* tile, const half8_t (&qhi)[KSTEPS],
                                            const half8_t (&qlo)[KSTEPS], int g, int n16) {
    const uint8_t* pa = tile + n16 * LDR + 16 * g;
    f32x4 h[2][2], r[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) h[u][0] = h[u][1] = r[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        const half8_t A0 = *reinterpret_cast<const half8_t*>(pa + 64 * s);
        const half8_t A1 = *reinterpret_cast<const half8_t*>(pa + 16 * LDR + 64 * s);
        h[0][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qhi[s], h[0][s & 1], 0, 0, 0);
        h[1][s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qhi[s], h[1][s & 1], 0, 0, 0);
        r[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qlo[s], r[0], 0, 0, 0);
        r[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qlo[s], r[1], 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) sn[u] = (h[u][0] + h[u][1]) + r[u];
}

__device__ __forceinline__ uint8_t* exch_slot(uint8_t* lds, int parity, int wave) {
    return lds + kBufs * TILE_BYTES + (parity * kWaves + wave) * EXCH_WAVE;
}

struct WaveState {
    half8_t qhi[KSTEPS], qlo[KSTEPS];   // own token, full width
    f32x4 acc[2][NT];                   // the pair's tokens, this wave's dims
    f32x4 sn[2];                        // own token's scores of the next tile
    float m_run, m_used, l_run;         // own token (lane = head n16)
    float qk_scale;
};

// The rescale a raised reference maximum asks for, before the context of
// tile j - 1 adds its weights: each token's accumulators times its heads'
// factors.  The accumulators make a round trip through this wave's own
// scratch in LDS and the multiply runs on the loaded copies: so no vector
// instruction ever takes the accumulators themselves, which lets them stay in
// the AGPRs where the matrix cores read and write them (a multiply in place
// makes the compiler keep or copy all of them through VGPRs on every tile).
// The compiler barriers keep it from forwarding the stored values past the
// LDS round trip.
__device__ __forceinline__ void rescale(WaveState& st, uint8_t* lds, const int* flags, int j, int lane, int wave,
                                        int g) {
    float* scr = reinterpret_cast<float*>(lds + SCR_OFF + wave * SCR_WAVE);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        if (flags[(wave & ~1) + u] != 0) {
            const uint8_t* ex = exch_slot(lds, (j - 1) & 1, (wave & ~1) + u);
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(ex + EX_ALPHA + 16 * g);   // heads 4g + i
#pragma unroll
            for (int t0 = 0; t0 < NT; t0 += 2) {
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    *reinterpret_cast<f32x4*>(scr + 4 * (64 * k + lane)) = st.acc[u][t0 + k];
                asm volatile("" ::: "memory");
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    f32x4* pk = reinterpret_cast<f32x4*>(scr + 4 * (64 * k + lane));
                    *pk = *pk * a4;
                }
                asm volatile("" ::: "memory");
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    st.acc[u][t0 + k] = *reinterpret_cast<const f32x4*>(scr + 4 * (64 * k + lane));
            }
        }
    }
}

// sched_barrier(0): the compiler moves no instruction across it.  The
// iteration below is written as a sequence of such sections, each holding one
// step's matrix-core instructions, the LDS reads for a step two or three ahead
// and a slice of the vector work, so that with one wave per SIMD the matrix
// cores always have issued work while LDS reads are in flight and the vector
// work fills the issue slots between them.
#define KVQ_SECTION() __builtin_amdgcn_sched_barrier(0)

// The two halves of iteration j (software pipeline, one barrier per
// iteration):
//   scores half: scores of tile j + 1 (16 k-steps x 4 MFMAs, the high and
//     residual query passes into separate accumulators, operands read three
//     steps ahead) with the online softmax of tile j sliced across the steps;
//     the weights, factors and flag of tile j are published for the partner;
//   context half: if any token of the workgroup raised its maximum on tile
//     j - 1, the rescale; then the context of tile j - 1 for both tokens of
//     the pair (pairs of dim tiles, 8 MFMAs each, operands read two pairs
//     ahead), with the conversion of tile j + 2 (into the buffer tile j - 2
//     used) and the loads of tile j + 3 sliced across the pairs, one row of
//     the wave's 8 per pair.
// Token pair 0 runs scores then context, pair 1 context then scores: the
// score half reads twice the LDS bytes per matrix-core instruction of the
// context half, so with the pairs in opposite halves the LDS demand of the
// workgroup stays even instead of peaking while all four waves score.
// MASK: rows at or past the own token's causal limit (vis rows of the chunk)
// are dropped from tile j.
template <bool MASK>
__device__ __forceinline__ void scores_half(WaveState& st, uint8_t* lds, int* flag_s, int j, int lane, int wave,
                                            int g, int n16, float w_scale, int vis) {
    const int rel0 = j * TR;
    const uint8_t* cur = lds + (j % kBufs) * TILE_BYTES;          // tile j: row scales
    const uint8_t* nxt = lds + ((j + 1) % kBufs) * TILE_BYTES;    // tile j + 1: score operands
    uint8_t* ex = exch_slot(lds, j & 1, wave);
    const f32x4 rsa = *reinterpret_cast<const f32x4*>(cur + TILE_F16 + 16 * g);
    const f32x4 rsb = *reinterpret_cast<const f32x4*>(cur + TILE_F16 + 64 + 16 * g);
    const uint8_t* pa = nxt + n16 * LDR + 16 * g;
    half8_t A[3][2];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        A[k][0] = *reinterpret_cast<const half8_t*>(pa + 64 * k);
        A[k][1] = *reinterpret_cast<const half8_t*>(pa + 16 * LDR + 64 * k);
    }
    // high pass in two chains (even / odd k-steps), residual pass in one
    f32x4 sh0 = {0.0f, 0.0f, 0.0f, 0.0f}, sh1 = sh0, sh2 = sh0, sh3 = sh0, sl0 = sh0, sl1 = sh0;
    float rs[8], sc[8], alpha = 1.0f, mu = 0.0f;
    bool need = false, started = false;
    half8_t phi, plo;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
        KVQ_SECTION();
        const int k = s % 3;
        if (s & 1) {
            sh2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k][0], st.qhi[s], sh2, 0, 0, 0);
            sh3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k][1], st.qhi[s], sh3, 0, 0, 0);
        } else {
            sh0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k][0], st.qhi[s], sh0, 0, 0, 0);
            sh1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k][1], st.qhi[s], sh1, 0, 0, 0);
        }
        sl0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k][0], st.qlo[s], sl0, 0, 0, 0);
        sl1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[k][1], st.qlo[s], sl1, 0, 0, 0);
        if (s + 3 < KSTEPS) {
            A[k][0] = *reinterpret_cast<const half8_t*>(pa + 64 * (s + 3));
            A[k][1] = *reinterpret_cast<const half8_t*>(pa + 16 * LDR + 64 * (s + 3));
        }
        if (s == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                rs[i] = rsa[i];
                rs[4 + i] = rsb[i];
                sc[i] = st.sn[0][i] * (rs[i] * st.qk_scale);
                sc[4 + i] = st.sn[1][i] * (rs[4 + i] * st.qk_scale);
            }
            if (MASK) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (rel0 + rho(g, e) >= vis) sc[e] = -INFINITY;
            }
        } else if (s == 1) {
            float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                               fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
            tmax = fmaxf(tmax, xor_lane<16>(tmax));
            tmax = fmaxf(tmax, xor_lane<32>(tmax));
            st.m_run = fmaxf(st.m_run, tmax);
        } else if (s == 2) {
            need = st.m_run > st.m_used + kRescaleSlack;
            // accumulators hold content only once a row was seen: before that zeros
            started = st.m_used != -INFINITY;
            const float m_new = need ? st.m_run : st.m_used;
            alpha = need ? __builtin_amdgcn_exp2f(st.m_used - m_new) : 1.0f;
            st.l_run *= alpha;
            st.m_used = m_new;
            mu = m_new == -INFINITY ? 0.0f : m_new;               // no row yet: p = 0
        } else if (s >= 3 && s < 7) {
#pragma unroll
            for (int e = 2 * (s - 3); e < 2 * (s - 3) + 2; ++e) {
                const float p = __builtin_amdgcn_exp2f(sc[e] - mu);
                st.l_run += p;
                // the rounded f32 product, then split: the pin (not volatile, so no
                // scheduling barrier) keeps the product from being fused into the
                // f16 conversion
                float w = p * (rs[e] * w_scale);
                asm("" : "+v"(w));
                const _Float16 h = (_Float16)w;
                phi[e] = h;
                plo[e] = (_Float16)(w - (float)h);
            }
        } else if (s == 7) {
            *reinterpret_cast<half8_t*>(ex + 16 * lane) = phi;
            *reinterpret_cast<half8_t*>(ex + EX_LO + 16 * lane) = plo;
            reinterpret_cast<float*>(ex + EX_ALPHA)[n16] = alpha;     // the 4 lanes of a head agree
            const bool flag = __builtin_amdgcn_ballot_w64(need && started) != 0ull;
            flag_s[kWaves * (j & 1) + wave] = flag ? 1 : 0;          // wave-uniform value
        }
    }
    KVQ_SECTION();
    st.sn[0] = (sh0 + sh2) + sl0;
    st.sn[1] = (sh1 + sh3) + sl1;
}

template <int FMT>
__device__ __forceinline__ void context_half(WaveState& st, TileRegs<FMT>& pf, const ChunkBufs& cb, uint8_t* lds,
                                             const uint32_t* lut, const u32x4& fl, int j, int tid, int lane,
                                             int wave, int half, int g, int n16) {
    constexpr int ROWB = TileFmt<FMT>::ROWB, W = TileFmt<FMT>::W;
    const int rel0 = j * TR;
    const uint8_t* prv = lds + ((j + 3) % kBufs) * TILE_BYTES;    // tile j - 1: context operands
    uint8_t* fill = lds + ((j + 2) % kBufs) * TILE_BYTES;         // tile j + 2
    if ((fl[0] | fl[1] | fl[2] | fl[3]) != 0u) {
        const int f[kWaves] = {(int)fl[0], (int)fl[1], (int)fl[2], (int)fl[3]};
        rescale(st, lds, f, j, lane, wave, g);
    }
    half8_t ph[2], pl[2];                   // weights of tile j - 1, both tokens of the pair
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const uint8_t* xp = exch_slot(lds, (j - 1) & 1, (wave & ~1) + u);
        ph[u] = *reinterpret_cast<const half8_t*>(xp + 16 * lane);
        pl[u] = *reinterpret_cast<const half8_t*>(xp + EX_LO + 16 * lane);
    }
    const uint8_t* pv = prv + (4 * g + (n16 >> 2)) * LDR + 2 * HALF * half + 8 * (n16 & 3);
    i16x4 V[3][4];                          // dim-tile pairs in flight: [pair][t0 h0, t0 h1, t1 h0, t1 h1]
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            V[k][c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4 __attribute__((address_space(3)))*)(pv + 32 * (2 * k + (c >> 1)) + (c & 1) * 16 * LDR));
    const int w4 = tid >> 6, l4 = tid & 63;
    uint8_t* dst = fill + 8 * w4 * LDR + 16 * l4;
    const int off = (rel0 + 3 * TR + 8 * w4) * ROWB + 4 * W * l4;   // tile j + 3, rows 8 * w4 + r
#pragma unroll
    for (int pr = 0; pr < NT / 2; ++pr) {
        KVQ_SECTION();
        const int k = pr % 3;
        if (pr + 2 < NT / 2) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                V[(pr + 2) % 3][c] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(pv + 32 * (2 * (pr + 2) + (c >> 1)) +
                                                                 (c & 1) * 16 * LDR));
        }
        half8_t B[2];
#pragma unroll
        for (int q = 0; q < 2; ++q)
            B[q] = __builtin_shufflevector(__builtin_bit_cast(half4_t, V[k][2 * q]),
                                           __builtin_bit_cast(half4_t, V[k][2 * q + 1]), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                st.acc[u][2 * pr + q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ph[u], B[q], st.acc[u][2 * pr + q], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                st.acc[u][2 * pr + q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl[u], B[q], st.acc[u][2 * pr + q], 0, 0, 0);
        // tile j + 2: row pr of this wave's 8 to f16, then its load for tile j + 3
        {
            const int r = pr;
            *reinterpret_cast<u32x4*>(dst + r * LDR) = row_f16<FMT>(pf.v[r], lut);
#pragma unroll
            for (int c = 0; c < W; ++c)
                pf.v[r][c] = __builtin_amdgcn_raw_buffer_load_b32(cb.codes, off + r * ROWB + 4 * c, 0, 0);
        }
        if (pr == NT / 2 - 1) {
            // threads t and t + 32k hold the same row's scale: same-value stores
            reinterpret_cast<float*>(fill + TILE_F16)[tid & (TR - 1)] = pf.s;
            pf.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 cb.scales, (rel0 + 3 * TR + (tid & 31)) * 4, 0, 0));
        }
    }
    KVQ_SECTION();
}

// Iterations [j, j_end), the same count and one barrier each for every wave.
template <int FMT, bool MASK, bool SCORES_FIRST>
__device__ __forceinline__ void run_tiles(WaveState& st, TileRegs<FMT>& pf, const ChunkBufs& cb, uint8_t* lds,
                                          const uint32_t* lut, int* flag_s, int j, int j_end, int tid, int lane,
                                          int wave, int half, int g, int n16, float w_scale, int vis) {
    for (; j < j_end; ++j) {
        // flags of tile j - 1 (published before the last barrier)
        const u32x4 fl = *reinterpret_cast<const u32x4*>(flag_s + kWaves * ((j - 1) & 1));
        if (SCORES_FIRST) {
            scores_half<MASK>(st, lds, flag_s, j, lane, wave, g, n16, w_scale, vis);
            context_half<FMT>(st, pf, cb, lds, lut, fl, j, tid, lane, wave, half, g, n16);
        } else {
            context_half<FMT>(st, pf, cb, lds, lut, fl, j, tid, lane, wave, half, g, n16);
            scores_half<MASK>(st, lds, flag_s, j, lane, wave, g, n16, w_scale, vis);
        }
        __syncthreads();
    }
}

// The decode's query, prepared once for every workgroup: per head (one wave,
// lane l holding dims 8l .. 8l+7), TQ4's q' = H D q (the encoder's sign
// flips, then the unnormalised Walsh-Hadamard transform: each butterfly leaves
// a + b in the lower and a - b in the upper element; strides 1 .. 4 inside the
// lane, 8 .. 256 by lane swaps), the headroom exponent eq of max |q'| and
// q' * 2^eq as f16 high part and f16 residual, in dim order, and the head's
// score factor 2^(-eq) (r / n) sm_scale log2(e).
template <int FMT>
__global__ __launch_bounds__(64) void k_prep_query(const float* __restrict__ q, uint64_t seed, float sm_scale,
                                                 _Float16* __restrict__ qhl, float* __restrict__ qks) {
    const int r = blockIdx.x;
    const int lane = threadIdx.x;
    const float* src = q + (int64_t)r * D + 8 * lane;
    const float4 u0 = *reinterpret_cast<const float4*>(src);
    const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
    float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    if constexpr (FMT == KVQ_TQ4) {
        const uint64_t wd = splitmix64_at(seed, (uint64_t)(lane >> 3));
        const int sh = 8 * (lane & 7);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((wd >> (sh + e)) & 1ull) v[e] = -v[e];
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
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    const int eq = headroom_exp(wave_max(m));
    half8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float xs = ldexpf(v[e], eq);
        hi[e] = (_Float16)xs;
        lo[e] = (_Float16)(xs - (float)hi[e]);
    }
    *reinterpret_cast<half8_t*>(qhl + (int64_t)(2 * r) * D + 8 * lane) = hi;
    *reinterpret_cast<half8_t*>(qhl + (int64_t)(2 * r + 1) * D + 8 * lane) = lo;
    if (lane == 0) qks[r] = ldexpf(1.0f, -eq - TileFmt<FMT>::LOG2_ROW_DIV) * sm_scale * kLog2e;
}

template <int FMT, int MODE>
__global__ __launch_bounds__(kThreads, 1) void k_mla_tiles(TileArgs a) {
    using F = TileFmt<FMT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float red_s[kWaves];
    __shared__ float lm_s[kWaves][2][16];
    __shared__ __attribute__((aligned(16))) int flag_s[2 * kWaves];  // [parity][wave]: a rescale is due
    __shared__ uint32_t lut_s[FMT == KVQ_TQ4 ? 256 : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave & 1;
    const int g = lane >> 4, n16 = lane & 15;
    int b = blockIdx.x;
    if (a.xcd_map) b = (b & 7) * (gridDim.x >> 3) + (b >> 3);
    // the units: prefill, tokens 4tg .. 4tg + 3 of head group hg (an idle token
    // past S repeats the last one); decode, head groups 0 .. 3 of token 0.
    // unit_row(u): the query / output row of the unit's head 0; unit_live(u):
    // whether its rows are written
    int chunk, hg = 0, tg = 0;
    int64_t lim_max, lim;                                   // rows the workgroup / own unit sees
    if constexpr (MODE == kPrefill) {
        const int n_hg = a.Hq / 16;
        hg = b % n_hg;
        chunk = (b / n_hg) % a.n_split;
        tg = b / (n_hg * a.n_split);
        const int own = kTok * tg + wave;
        const int tok = own < a.S ? own : a.S - 1;
        const int last_tok = (kTok * tg + kTok - 1 < a.S) ? kTok * tg + kTok - 1 : a.S - 1;
        lim_max = a.pos0 + last_tok + 1;
        lim = a.pos0 + tok + 1;
    } else {
        chunk = b;
        lim_max = lim = a.T;
    }
    auto unit_row = [&](int u) -> int64_t {
        if constexpr (MODE == kPrefill) {
            const int t = kTok * tg + u;
            return (int64_t)(t < a.S ? t : a.S - 1) * a.Hq + hg * 16;
        } else {
            return (int64_t)u * 16;
        }
    };
    auto unit_live = [&](int u) -> bool { return MODE == kPrefill ? kTok * tg + u < a.S : true; };
    const int64_t c0 = (int64_t)chunk * a.chunk;
    const int64_t c1 = (c0 + a.chunk < lim_max) ? c0 + a.chunk : lim_max;
    const int n_tiles = c1 > c0 ? (int)((c1 - c0 + TR - 1) / TR) : 0;
    const int n_rows32 = c1 > c0 ? (int)(c1 - c0) : 0;
    const int vis = lim <= c0 ? 0 : (lim - c0 < n_rows32 ? (int)(lim - c0) : n_rows32);   // own unit's rows
    ChunkBufs cbuf;
    cbuf.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.codes + c0 * F::ROWB), (short)0,
                                                   n_rows32 * F::ROWB, kBufWord3);
    cbuf.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.scales + c0), (short)0,
                                                    n_rows32 * 4, kBufWord3);

    // ---- loads in the order they are needed: the first round of row factors
    // (weight pre-scale), tiles 0 and 1, then the own query (full width) ----
    // Row factors past the chunk read as zeros through the buffer resource.
    float f0[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
        f0[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cbuf.scales, (tid + u * kThreads) * 4,
                                                                               0, 0));
    TileRegs<FMT> pf, pf1;
    load_tile<FMT>(pf, cbuf, 0, tid);
    load_tile<FMT>(pf1, cbuf, TR, tid);
    // lane (n16, g): head n16, dims 32s + 8g + [0, 8) for s < 16.  Prefill: the
    // f32 query, split below; decode: the prepared operands and score factor
    WaveState st;
    f32x4 xq[KSTEPS][2];
    if constexpr (MODE == kPrefill) {
        const float* src = a.q + (unit_row(wave) + n16) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            xq[s][0] = *reinterpret_cast<const f32x4*>(src + 32 * s);
            xq[s][1] = *reinterpret_cast<const f32x4*>(src + 32 * s + 4);
        }
    } else {
        const int64_t head = unit_row(wave) + n16;
        const _Float16* src = a.qhl + 2 * head * D + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            st.qhi[s] = *reinterpret_cast<const half8_t*>(src + 32 * s);
            st.qlo[s] = *reinterpret_cast<const half8_t*>(src + D + 32 * s);
        }
        st.qk_scale = a.qks[head];
    }

    if constexpr (FMT == KVQ_TQ4) {
        // byte -> (f16 level of the low nibble, f16 level of the high nibble)
        // (the 16 levels are read as uniform values and selected per lane)
        const int nlo = tid & 15, nhi = tid >> 4;
        float llo = a.level[0], lhi = a.level[0];
#pragma unroll
        for (int k = 1; k < 16; ++k) {
            llo = nlo == k ? a.level[k] : llo;
            lhi = nhi == k ? a.level[k] : lhi;
        }
        lut_s[tid] = f16_bits_rne(llo) | (f16_bits_rne(lhi) << 16);
    }

    // ---- weight pre-scale: max row factor over the rows the workgroup sees ----
    float smax = fmaxf(fmaxf(f0[0], f0[1]), fmaxf(f0[2], f0[3]));
    for (int r0 = tid + 4 * kThreads; r0 < n_rows32; r0 += 4 * kThreads) {
        float f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            f[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(cbuf.scales,
                                                                                  (r0 + u * kThreads) * 4, 0, 0));
        smax = fmaxf(smax, fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])));
    }
    smax = wave_max(smax);
    if (lane == 0) red_s[wave] = smax;
    // no tile -1: zero weights and flags in the slots the first iteration reads,
    // and zero rows in the buffer its context step reads (0 * NaN bits would not be 0)
    for (int i = tid; i < TILE_F16 / 16; i += kThreads)
        reinterpret_cast<u32x4*>(lds + (kBufs - 1) * TILE_BYTES)[i] = u32x4{0u, 0u, 0u, 0u};
    {
        uint8_t* ex = exch_slot(lds, 1, wave);
        *reinterpret_cast<u32x4*>(ex + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(ex + EX_LO + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        if (lane == 0) flag_s[kWaves + wave] = 0;
    }
    if constexpr (MODE == kPrefill) {
        // the head's max over the full width, then q * 2^eq as f16 high / residual
        float hm = 0.0f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) hm = fmaxf(hm, fabsf(xq[s][e >> 2][e & 3]));
        hm = fmaxf(hm, xor_lane<16>(hm));
        hm = fmaxf(hm, xor_lane<32>(hm));
        const int eq = headroom_exp(hm);
        st.qk_scale = ldexpf(1.0f, -eq - F::LOG2_ROW_DIV) * a.sm_scale * kLog2e;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xs = ldexpf(xq[s][e >> 2][e & 3], eq);
                const _Float16 h = (_Float16)xs;
                st.qhi[s][e] = h;
                st.qlo[s][e] = (_Float16)(xs - (float)h);
            }
    }
    st.m_run = st.m_used = -INFINITY;
    st.l_run = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) st.acc[u][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // ---- pipeline fill: tiles 0 and 1 converted, tile 2 in flight ----
    if constexpr (FMT == KVQ_TQ4) __syncthreads();          // the byte table is complete
    store_tile<FMT>(lds, pf, tid, lut_s);
    load_tile<FMT>(pf, cbuf, 2 * TR, tid);
    store_tile<FMT>(lds + TILE_BYTES, pf1, tid, lut_s);
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) smax = fmaxf(smax, red_s[w]);
    const int ew = headroom_exp(smax) - kWeightShift;
    const float w_scale = ldexpf(1.0f, ew);
    tile_scores(st.sn, lds, st.qhi, st.qlo, g, n16);

    // iterations 0..n_tiles: iteration n_tiles only finishes the context of the
    // last tile (its softmax step sees a tile past every limit, fully masked)
    const int j_mask = vis / TR < n_tiles ? vis / TR : n_tiles;
    // Pair 0 runs each iteration's halves in the order scores, context; pair 1
    // in the order context, scores.  Each order is its own copy of the whole
    // sweep and the output (so each gets its own register assignment);
    // barriers count per workgroup, not per code location.
    auto sweep = [&](auto order) {
        constexpr bool SF = decltype(order)::value;
        run_tiles<FMT, false, SF>(st, pf, cbuf, lds, lut_s, flag_s, 0, j_mask, tid, lane, wave, half, g, n16,
                                  w_scale, vis);
        run_tiles<FMT, true, SF>(st, pf, cbuf, lds, lut_s, flag_s, j_mask, n_tiles + 1, tid, lane, wave, half, g,
                                 n16, w_scale, vis);

        // ---- output.  Own unit's l and m to the pair; each wave then writes
        // acc * 2^-(ew + row div) / l for the pair's units on its dims (one
        // chunk), or that partial without / l and (m, l); staged for 16-byte
        // stores ----
        float l = st.l_run;
        l += xor_lane<16>(l);
        l += xor_lane<32>(l);
        if (g == 0) {
            lm_s[wave][0][n16] = l;
            lm_s[wave][1][n16] = st.m_used;
        }
        __syncthreads();
        const int64_t n_qrows = (int64_t)a.S * a.Hq;
        const float unscale = ldexpf(1.0f, -ew - F::LOG2_ROW_DIV);
        float* ost = reinterpret_cast<float*>(lds) + wave * 2 * 16 * OUT_ROW;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int src_wave = (wave & ~1) + u;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lh = lm_s[src_wave][0][4 * g + i];
                const float f = a.n_split == 1 ? unscale / lh : unscale;
#pragma unroll
                for (int t = 0; t < NT; ++t) ost[(16 * u + 4 * g + i) * OUT_ROW + 16 * t + n16] = st.acc[u][t][i] * f;
            }
        }
        if (unit_live(wave) && g == 0) {
            const int64_t qrow = unit_row(wave) + n16;
            if (a.n_split == 1) {
                if (a.lse != nullptr) a.lse[qrow] = (st.m_used + log2f(l)) * 0.69314718055994531f;
            } else {
                float* ml = a.part_ml + ((int64_t)chunk * n_qrows + qrow) * 2;
                ml[0] = st.m_used;
                ml[1] = l;
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pu = (wave & ~1) + u;
            if (unit_live(pu)) {
                // a wave's LDS operations complete in issue order: its staged rows are in place
                // 16 heads x 256 dims of this unit: 16 f32x4 per lane
                float* dst = (a.n_split == 1 ? a.out : a.part_acc + (int64_t)chunk * n_qrows * D) +
                             unit_row(pu) * D + HALF * half;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int idx = lane + 64 * k;              // 0..1023: head idx/64, dims 4*(idx%64)
                    const int h = idx >> 6, dd = 4 * (idx & 63);
                    const f32x4 v = *reinterpret_cast<const f32x4*>(ost + (16 * u + h) * OUT_ROW + dd);
                    *reinterpret_cast<f32x4*>(dst + (int64_t)h * D + dd) = v;
                }
            }
        }
    };
    if (wave < 2)
        sweep(std::true_type{});
    else
        sweep(std::false_type{});
}

template <int FMT, int MODE>
hipError_t launch_tiles(TileArgs& a, int blocks, hipStream_t s) {
    a.xcd_map = (blocks % 8 == 0) ? 1 : 0;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_dyn_lds_once(reinterpret_cast<const void*>(&k_mla_tiles<FMT, MODE>), kDynLds, lds_set);
    if (e != hipSuccess) return e;
    k_mla_tiles<FMT, MODE><<<blocks, kThreads, kDynLds, s>>>(a);
    return hipGetLastError();
}

TileArgs tile_args(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq, int32_t S, int64_t pos0,
                   float sm_scale, float* part_acc, float* part_ml, float* out, float* lse) {
    TileArgs a;
    a.codes = kv.codes;
    a.scales = reinterpret_cast<const float*>(kv.scales);
    a.q = q;
    a.sm_scale = sm_scale;
    a.T = kv.n_rows;
    a.Hq = Hq;
    a.S = S;
    a.pos0 = pos0;
    a.out = out;
    a.lse = lse;
    a.chunk = p.chunk;
    a.n_split = p.n_split;
    a.part_acc = part_acc;
    a.part_ml = part_ml;
    a.xcd_map = 0;
    const Codebook16& cb = codebook16();
    for (int i = 0; i < 16; ++i) a.level[i] = cb.level[i];
    a.qhl = nullptr;
    a.qks = nullptr;
    return a;
}

}  // namespace

// From 8 tokens on; below that one workgroup per (token, head group, chunk) of
// the decode kernel is faster (measured at T = 32768, 64 heads: S = 2 and 4
// take 34 and 54 us there against 48 and 62 us here, S = 8 and 16 are even,
// S = 64 is 5 % faster here, a 512-token prefill 17 %)
bool mla_prefill_kv8_eligible(const kvq_cache& kv, int32_t Hq, int32_t S) {
    return kv.fmt == KVQ_FP8 && kv.d == D && kv.d_rope == 0 && Hq % 16 == 0 && S >= 8;
}

// about one workgroup per CU: 256 / (token groups x head groups) chunks in
// whole tiles, or one chunk when the prefill alone fills the GPU
void mla_prefill_kv8_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p) {
    const int64_t groups = (int64_t)((S + kTok - 1) / kTok) * (Hq / 16);
    const int64_t T = kv.n_rows;
    int64_t want = (256 + groups - 1) / groups;
    int64_t chunk = (T + want - 1) / want;
    chunk = ((chunk + TR - 1) / TR) * TR;
    if (chunk > kMaxChunk) chunk = kMaxChunk;               // 32-bit buffer offsets in the kernel
    p.path = 1;
    p.chunk = chunk;
    p.n_split = (int32_t)((T + chunk - 1) / chunk);
    p.n_qrows = Hq * S;
    p.heads_per_blk = 16;
    p.n_qgroups = (int32_t)groups;
    p.log2_domain = 1;
    p.ws_bytes = (size_t)p.n_split * p.n_qrows * (D + 2) * sizeof(float);
}

hipError_t launch_mla_prefill_kv8(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                                  int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                                  float* part_ml, float* out, float* lse, hipStream_t s) {
    TileArgs a = tile_args(kv, p, q, Hq, S, pos0, sm_scale, part_acc, part_ml, out, lse);
    const int blocks = ((S + kTok - 1) / kTok) * (Hq / 16) * p.n_split;
    return launch_tiles<KVQ_FP8, kPrefill>(a, blocks, s);
}

// TQ4 decode of one token with 64 heads over a long cache: each row is
// decoded once for the 4 head groups (the per-head-group kernel decodes it
// once per group); shorter caches keep that kernel, whose 4x more workgroups
// fill the GPU sooner
bool mla_decode64_eligible(const kvq_cache& kv, int32_t Hq, int32_t S) {
    const int64_t min_rows = kv.fmt == KVQ_TQ4 ? kDecode64MinRows : kDecode64MinRowsKv8;
    return (kv.fmt == KVQ_TQ4 || kv.fmt == KVQ_FP8) && kv.d == D && kv.d_rope == 0 && Hq == 64 && S == 1 &&
           kv.n_rows >= min_rows;
}

// about one workgroup per CU: 256 chunks in whole tiles
void mla_decode64_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p) {
    const int64_t T = kv.n_rows;
    int64_t chunk = (T + 255) / 256;
    chunk = ((chunk + TR - 1) / TR) * TR;
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    p.path = 1;
    p.chunk = chunk;
    p.n_split = (int32_t)((T + chunk - 1) / chunk);
    p.n_qrows = Hq * S;
    p.heads_per_blk = 64;
    p.n_qgroups = 1;
    p.log2_domain = 1;
    // partials, then the prepared query (f16 high and residual) and its factors
    p.ws_bytes = (size_t)p.n_split * p.n_qrows * (D + 2) * sizeof(float) + (size_t)Hq * 2 * D * 2 +
                 (size_t)Hq * sizeof(float);
}

hipError_t launch_mla_decode64(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq, int32_t S,
                               int64_t pos0, float sm_scale, float* part_acc, float* part_ml, float* out,
                               float* lse, hipStream_t s) {
    TileArgs a = tile_args(kv, p, q, Hq, S, pos0, sm_scale, part_acc, part_ml, out, lse);
    _Float16* qhl = reinterpret_cast<_Float16*>(part_ml + (size_t)p.n_split * p.n_qrows * 2);   // 16-byte aligned
    float* qks = reinterpret_cast<float*>(qhl + (size_t)Hq * 2 * D);
    if (kv.fmt == KVQ_TQ4)
        k_prep_query<KVQ_TQ4><<<Hq, 64, 0, s>>>(q, kv.rot_seed, sm_scale, qhl, qks);
    else
        k_prep_query<KVQ_FP8><<<Hq, 64, 0, s>>>(q, 0, sm_scale, qhl, qks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.qhl = qhl;
    a.qks = qks;
    if (kv.fmt == KVQ_TQ4) return launch_tiles<KVQ_TQ4, kDecode>(a, p.n_split, s);
    return launch_tiles<KVQ_FP8, kDecode>(a, p.n_split, s);
}

}  // namespace kvq
