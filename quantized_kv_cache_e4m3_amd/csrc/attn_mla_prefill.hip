// KV8 chunked prefill for the MLA latent (d = 512, heads in groups of 16) on
// the gfx950 matrix cores, in flash-attention tiles shared by 4 tokens.
//
// [colibri #553] "What's in it" / [colibri #399] "Commits" item 2: the rows
// are consumed as they are stored (fp8 e4m3 values, the f32 row scale outside
// the dot product) and the latent row is both key and value; token s of the
// prefill attends rows t <= pos0 + s.
//
// Both products run on v_mfma_f32_16x16x32_f16 with exact f16 operands: e4m3
// values are exact in f16, and the f32 side (query, weights p * row scale) is
// split into an f16 high part and an f16 residual multiplied in two passes,
// pre-scaled by powers of two.
//
// Work layout.  Workgroup = (4 consecutive tokens, 16 heads), 8 waves = 4
// pairs; pair p serves token 4*tg + p and its two waves split the latent
// width (dims [256h, 256h + 256)), as in the decode kernel.  All pairs walk
// the same 32-row tiles: each tile is loaded once (its fp8 rows prefetched one
// tile ahead into registers, 32 bytes per thread), converted once to f16 by
// the whole workgroup into a double-buffered LDS tile (1040-byte rows), and
// read by every pair: score operands as 16-byte row reads, context operands by
// ds_read_b64_tr_b16 (8 rows of one dim per lane, in the order rho(g, e) in
// which the score accumulators already hold the weights).  So the fp8 -> f16
// conversion is paid once per row for 64 query rows instead of once per pair.
// Per tile: convert, barrier, scores, partner exchange through LDS, barrier,
// online softmax with the token's causal limit, context.  With one chunk
// (a long prefill) each pair writes its token's normalized output and lse;
// otherwise the rows are split into chunks (grid = token groups x chunks x
// head groups) and each pair writes an (m, l, acc) partial for the combine
// step.
#include <math.h>

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
constexpr int KSTEPS = HALF / 32;       // 8 score k-steps per wave
constexpr int NT = HALF / 16;           // 16 context dim tiles per wave
constexpr int kWaves = 8, kPairs = 4;   // pairs = tokens per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int LDR = 2 * D + 16;         // f16 tile row stride (bytes)
constexpr int TILE_BYTES = TR * LDR;
constexpr int EXCH_BYTES = 2 * kWaves * 512 * 4;    // double-buffered partial scores
constexpr int kLoopLds = 2 * TILE_BYTES + EXCH_BYTES;
constexpr int OUT_ROW = HALF + 4;       // output staging row (floats)
constexpr int kOutLds = kWaves * 16 * OUT_ROW * 4;
constexpr int kDynLds = kLoopLds > kOutLds ? kLoopLds : kOutLds;
static_assert(kDynLds <= 160 * 1024 - 1024, "LDS budget");
constexpr float kRescaleSlack = 8.0f;   // log2 units: p <= 2^8 between rescales
constexpr int kWeightShift = 7;         // 2^ew * (max row scale) in [2^6, 2^7): weights < 2^15
constexpr float kLog2e = 1.4426950408889634f;

struct PrefillArgs {
    const uint8_t* codes;   // [T][D] e4m3
    const float* scales;    // [T]
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
};

__device__ __forceinline__ int headroom_exp(float x) {
    if (!(x > 0.0f)) return 0;
    int k;
    (void)frexpf(x, &k);
    return 14 - k;
}

// row of the tile held in context slot e of lane group g
__device__ __forceinline__ int rho(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

struct TileRegs {
    u32x4 v[2];             // thread t: 32 fp8 bytes at 32*(t%16) of row t/16
    float s[8];             // row scales of the lane's context rows rho(g, 0..7)
};

// The chunk's rows are read through buffer resources whose base is the
// chunk's first row and whose range ends at the last row the token group
// sees: a row past it reads as zeros without a memory access (such rows are
// masked by the causal limit), so offsets are 32-bit rows inside the chunk
// (the plan caps the chunk) and nothing is clamped per row.
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 (32-bit data format)
constexpr int64_t kMaxChunk = int64_t{1} << 21;
struct ChunkBufs {
    __amdgpu_buffer_rsrc_t codes, scales;
};

__device__ __forceinline__ void load_tile(TileRegs& r, const ChunkBufs& b, int rel0, int tid, int g) {
    const int off = (rel0 + (tid >> 4)) * D + 32 * (tid & 15);
    r.v[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b.codes, off, 0, 0));
    r.v[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b.codes, off + 16, 0, 0));
    const int soff = (rel0 + 4 * g) * 4;
    const f32x4 s0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.scales, soff, 0, 0));
    const f32x4 s1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(b.scales, soff + 64, 0, 0));
    r.s[0] = s0[0]; r.s[1] = s0[1]; r.s[2] = s0[2]; r.s[3] = s0[3];
    r.s[4] = s1[0]; r.s[5] = s1[1]; r.s[6] = s1[2]; r.s[7] = s1[3];
}

__global__ __launch_bounds__(kThreads, 1) void k_mla_prefill_kv8(PrefillArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float hmax_s[kWaves][16];
    __shared__ float red_s[kWaves];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave >> 1, half = wave & 1;
    const int g = lane >> 4, n16 = lane & 15;
    const int n_hg = a.Hq / 16;
    int b = blockIdx.x;
    if (a.xcd_map) b = (b & 7) * (gridDim.x >> 3) + (b >> 3);
    const int hg = b % n_hg;
    const int chunk = (b / n_hg) % a.n_split, tg = b / (n_hg * a.n_split);
    const int tok = kPairs * tg + pair;
    const bool active = tok < a.S;                          // wave-uniform
    const int last_tok = (kPairs * tg + kPairs - 1 < a.S) ? kPairs * tg + kPairs - 1 : a.S - 1;
    const int64_t lim_max = a.pos0 + last_tok + 1;          // rows any token of the group sees
    const int64_t lim = a.pos0 + tok + 1;                   // this pair's causal limit
    const int64_t c0 = (int64_t)chunk * a.chunk;
    const int64_t c1 = (c0 + a.chunk < lim_max) ? c0 + a.chunk : lim_max;
    const int n_tiles = c1 > c0 ? (int)((c1 - c0 + TR - 1) / TR) : 0;
    const int n_rows32 = c1 > c0 ? (int)(c1 - c0) : 0;
    // this pair's causal limit as a row of the chunk, in [0, n_rows32]
    const int lim_rel = lim <= c0 ? 0 : (lim - c0 < n_rows32 ? (int)(lim - c0) : n_rows32);
    ChunkBufs cbuf;
    cbuf.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.codes + c0 * D), (short)0,
                                                   n_rows32 * D, kBufWord3);
    cbuf.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.scales + c0), (short)0,
                                                    n_rows32 * 4, kBufWord3);
    const int64_t qrow = (int64_t)(active ? tok : 0) * a.Hq + hg * 16 + n16;   // this lane's head

    // ---- loads in the order they are needed: query slice, first tile ----
    // lane (n16, g): head n16, dims 256*half + 32s + 8g + [0, 8) for s < 8
    float xq[KSTEPS][8];
    {
        const float* src = a.q + qrow * D + HALF * half + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const float4 u0 = *reinterpret_cast<const float4*>(src + 32 * s);
            const float4 u1 = *reinterpret_cast<const float4*>(src + 32 * s + 4);
            xq[s][0] = u0.x; xq[s][1] = u0.y; xq[s][2] = u0.z; xq[s][3] = u0.w;
            xq[s][4] = u1.x; xq[s][5] = u1.y; xq[s][6] = u1.z; xq[s][7] = u1.w;
        }
    }
    TileRegs pf;
    if (n_tiles > 0) load_tile(pf, cbuf, 0, tid, g);

    // ---- weight pre-scale: max row scale over the rows the group sees ----
    float smax = 0.0f;
    for (int64_t t0 = c0 + tid; t0 < c1; t0 += 4 * kThreads) {
        float f[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) f[u] = t0 + u * kThreads < c1 ? a.scales[t0 + u * kThreads] : 0.0f;
        smax = fmaxf(smax, fmaxf(fmaxf(f[0], f[1]), fmaxf(f[2], f[3])));
    }
    smax = wave_max(smax);
    float hm = 0.0f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) hm = fmaxf(hm, fabsf(xq[s][e]));
    hm = fmaxf(hm, xor_lane<16>(hm));
    hm = fmaxf(hm, xor_lane<32>(hm));
    if (g == 0) hmax_s[wave][n16] = hm;
    if (lane == 0) red_s[wave] = smax;
    __syncthreads();
    // the head's max over both halves of the pair, then q * 2^eq as f16 high / residual
    const int eq = headroom_exp(fmaxf(hmax_s[wave][n16], hmax_s[wave ^ 1][n16]));
    const float qk_scale = ldexpf(1.0f, -eq) * a.sm_scale * kLog2e;
    half8_t qhi[KSTEPS], qlo[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xs = ldexpf(xq[s][e], eq);
            const _Float16 h = (_Float16)xs;
            qhi[s][e] = h;
            qlo[s][e] = (_Float16)(xs - (float)h);
        }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) smax = fmaxf(smax, red_s[w]);
    const float w_scale = ldexpf(1.0f, headroom_exp(smax) - kWeightShift);

    float* exch = reinterpret_cast<float*>(lds + 2 * TILE_BYTES);
    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, m_used = -INFINITY, l_run = 0.0f;

    for (int j = 0; j < n_tiles; ++j) {
        const int rel0 = j * TR;                        // first row of the tile in the chunk
        uint8_t* const tile = lds + (j & 1) * TILE_BYTES;
        // ---- convert the tile once (32 fp8 -> 32 f16 per thread) ----
        {
            uint8_t* dst = tile + (tid >> 4) * LDR + 64 * (tid & 15);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                u32x4 h0, h1;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = pf.v[k][c];
                    const half2_t lo2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
                    const half2_t hi2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
                    if (c < 2) {
                        h0[2 * c] = __builtin_bit_cast(uint32_t, lo2);
                        h0[2 * c + 1] = __builtin_bit_cast(uint32_t, hi2);
                    } else {
                        h1[2 * (c - 2)] = __builtin_bit_cast(uint32_t, lo2);
                        h1[2 * (c - 2) + 1] = __builtin_bit_cast(uint32_t, hi2);
                    }
                }
                *reinterpret_cast<u32x4*>(dst + 32 * k) = h0;
                *reinterpret_cast<u32x4*>(dst + 32 * k + 16) = h1;
            }
        }
        float srow[8], wrow[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            srow[e] = pf.s[e] * qk_scale;
            wrow[e] = pf.s[e] * w_scale;
        }
        if (j + 1 < n_tiles) load_tile(pf, cbuf, rel0 + TR, tid, g);
        __syncthreads();                                // tile j converted

        // ---- partial scores over this wave's half of the dims ----
        float* mine = exch + ((j & 1) * kWaves + wave) * 512 + lane * 8;
        if (active) {
            f32x4 s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
            f32x4 s0l = {0.0f, 0.0f, 0.0f, 0.0f}, s1l = {0.0f, 0.0f, 0.0f, 0.0f};
            const uint8_t* pa = tile + n16 * LDR + 2 * (HALF * half + 8 * g);
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s) {
                const half8_t A0 = *reinterpret_cast<const half8_t*>(pa + 64 * s);
                const half8_t A1 = *reinterpret_cast<const half8_t*>(pa + 16 * LDR + 64 * s);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qhi[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qhi[s], s1, 0, 0, 0);
                s0l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A0, qlo[s], s0l, 0, 0, 0);
                s1l = __builtin_amdgcn_mfma_f32_16x16x32_f16(A1, qlo[s], s1l, 0, 0, 0);
            }
            s0 += s0l;
            s1 += s1l;
            *reinterpret_cast<f32x4*>(mine) = s0;
            *reinterpret_cast<f32x4*>(mine + 4) = s1;
        }
        __syncthreads();                                // partial scores exchanged
        if (!active) continue;
        const float* other = exch + ((j & 1) * kWaves + (wave ^ 1)) * 512 + lane * 8;
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(other);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(other + 4);
        const f32x4 m0 = *reinterpret_cast<const f32x4*>(mine);
        const f32x4 m1 = *reinterpret_cast<const f32x4*>(mine + 4);
        float sc[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // the same sum in both waves of the pair (a + b == b + a)
            sc[i] = (m0[i] + o0[i]) * srow[i];
            sc[4 + i] = (m1[i] + o1[i]) * srow[4 + i];
        }
        if (rel0 + TR > lim_rel) {                      // causal limit inside this tile
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (rel0 + rho(g, e) >= lim_rel) sc[e] = -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = fmaxf(tmax, xor_lane<16>(tmax));
        tmax = fmaxf(tmax, xor_lane<32>(tmax));
        if (tmax == -INFINITY) continue;                // tile entirely past this token's rows
        m_run = fmaxf(m_run, tmax);
        const bool need = m_run > m_used + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
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
            const float w = opaque(p * wrow[e]);      // rounded f32 product, then split
            const _Float16 h = (_Float16)w;
            phi[e] = h;
            plo[e] = (_Float16)(w - (float)h);
        }
        // ---- context over this wave's 256 dims ----
        const uint8_t* pv = tile + (4 * g + (n16 >> 2)) * LDR + 2 * HALF * half + 8 * (n16 & 3);
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

    // ---- output: acc * 2^-ew / l for the pair's token (one chunk), or the
    // partial acc * 2^-ew and (m, l); staged for 16-byte stores ----
    l_run += xor_lane<16>(l_run);
    l_run += xor_lane<32>(l_run);
    __syncthreads();                                    // tiles and exchange consumed
    float* ost = reinterpret_cast<float*>(lds) + wave * 16 * OUT_ROW;
    const float inv = 1.0f / w_scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float lh = __shfl(l_run, 4 * g + i);      // head 4g + i's l (lane 4g + i holds it)
        const float f = !active ? 0.0f : (a.n_split == 1 ? inv / lh : inv);
#pragma unroll
        for (int t = 0; t < NT; ++t) ost[(4 * g + i) * OUT_ROW + 16 * t + n16] = acc[t][i] * f;
    }
    const int64_t n_qrows = (int64_t)a.S * a.Hq;
    if (active && half == 0 && g == 0) {
        if (a.n_split == 1) {
            if (a.lse != nullptr) a.lse[qrow] = (m_used + log2f(l_run)) * 0.69314718055994531f;
        } else {
            float* ml = a.part_ml + ((int64_t)chunk * n_qrows + qrow) * 2;
            ml[0] = m_used;
            ml[1] = l_run;
        }
    }
    if (active) {
        // a wave's LDS operations complete in issue order: its staged rows are in place
        // 16 heads x 256 dims of this wave: 16 f32x4 per lane
        float* dst = (a.n_split == 1 ? a.out : a.part_acc + (int64_t)chunk * n_qrows * D) +
                     ((int64_t)tok * a.Hq + hg * 16) * D + HALF * half;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const int idx = lane + 64 * k;              // 0..1023: head idx/64, dims 4*(idx%64)
            const int h = idx >> 6, dd = 4 * (idx & 63);
            const f32x4 v = *reinterpret_cast<const f32x4*>(ost + h * OUT_ROW + dd);
            *reinterpret_cast<f32x4*>(dst + (int64_t)h * D + dd) = v;
        }
    }
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
    const int64_t groups = (int64_t)((S + kPairs - 1) / kPairs) * (Hq / 16);
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
    PrefillArgs a;
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
    const int blocks = ((S + kPairs - 1) / kPairs) * (Hq / 16) * p.n_split;
    a.xcd_map = (blocks % 8 == 0) ? 1 : 0;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_dyn_lds_once(reinterpret_cast<const void*>(&k_mla_prefill_kv8), kDynLds, lds_set);
    if (e != hipSuccess) return e;
    k_mla_prefill_kv8<<<blocks, kThreads, kDynLds, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvq
