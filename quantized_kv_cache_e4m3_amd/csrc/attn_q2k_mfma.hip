// GQA decode attention over a q2k cache (d = 256 per KV head, 8 query heads
// per KV head) on the gfx950 matrix cores.
//
// [Strata #2318] "Summary" items 1-3 and "Why per-channel K and per-token V":
// bulk K is a 2-bit level per (cell, channel) times an fp16 scale per
// (32-cell group, channel); bulk V is q4_0, (code - 8) times an fp16 scale
// per (cell, 32-channel block); the first n_sink cells and the last n_window
// cells read exact fp16 copies instead.  The cache is read as stored: each
// 32-cell group is decoded once into LDS and consumed there.
//
// Both products are MFMA v_mfma_f32_16x16x32_f16 with exact f16 operands:
//   scores   S[cell, 2h+p] = sum_c K[cell, c] * Qp[h][c]      (p: query hi/lo)
//   context  C[2h+p, c]   += sum_cell Pp[h][cell] * V[cell, c] (p: weight hi/lo)
// The 8 query heads fill the 16 MFMA columns (rows) twice: once with the f16
// high part of the pre-scaled query (weight), once with its f16 residual, so
// one MFMA carries both terms of the split; the two columns are added after
// the score product and the two accumulator rows after the last chunk.  K and
// V values are not f16 numbers (level * scale has 22 significant bits,
// (code - 8) * d has 15), so each is staged as an exact f16 pair hi + lo
// (v_pk_mul_f16 gives hi, v_pk_fma_f16 the exact residual) and multiplied
// twice.  Overlay K cells are fp16 already and are staged as they are
// (residual 0).  The staged values carry power-of-two pre-scales chosen from
// the stored values so that nothing overflows f16: one per group for the bulk
// K (its scores are scaled back per cell), one per wave for V, set by the
// wave's first group and lowered (rescaling the accumulator by the exact power
// of two) when a later group, bulk or overlay, holds larger values.
//
// Work layout.  Workgroup = (slice of 32-cell groups, KV head), 4 waves; slice
// j of n holds groups j, j+n, j+2n, ... (the overlay groups at both ends of
// the cache land in different slices); wave w takes the slice's groups w,
// w+4, ... with a private online softmax and private accumulators, merged in
// LDS at the end into one (m, l, acc) partial per slice (m in log2 units) for
// the combine kernel.  Per group a wave
//   1. stages K hi/lo as [cell][channel] f16 (lane: 4 channels x 32 cells; the
//      2-bit codes of 4 cells of 4 channels are transposed with v_perm, a
//      4-entry byte table gives the levels),
//   2. runs the score MFMAs (K rows by ds_read_b128, query from registers),
//   3. updates the online softmax (rows of a lane: cells rho(g, e) = 16*(e/4)
//      + 4g + e%4, the context MFMA's k order),
//   4. stages V hi/lo as [cell][channel] f16 into the same LDS (raw 144-byte
//      cell rows first; lane: 4 (cell, block) pairs, nibbles to f16 through
//      the 0x6400 exponent trick),
//   5. runs the context MFMAs (V operand by ds_read_b64_tr_b16).
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 256;                  // channels per KV head
constexpr int G = 8;                    // query heads per KV head
constexpr int CELLS = 32;               // cells per group
constexpr int NBLK = D / 32;            // q4_0 blocks per cell
constexpr int KSTEPS = D / 32;          // score k-steps
constexpr int NT = D / 16;              // context dim tiles
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int ROW = 2 * D + 16;         // LDS bytes per staged f16 row (padded)
constexpr int BUF = CELLS * ROW;        // one staged [cell][channel] f16 matrix
constexpr int RAWROW = NBLK * 18;       // bytes of one cell's V blocks for one KV head
constexpr int RAW = CELLS * RAWROW;
constexpr int WAVE_LDS = 2 * BUF + RAW;
constexpr int kDynLds = kWaves * WAVE_LDS;   // 153600 B
constexpr int NPIECE = CELLS * RAWROW / 16;  // 288 16-byte pieces of a group's V rows
constexpr float kRescaleSlack = 1.0f;   // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPScale = 4096.0f;      // weights p <= 2 staged as p * 2^12 (< 2^14)

static_assert(kDynLds <= 160 * 1024 - 2048, "LDS budget");
static_assert(kWaves * 16 * D * 4 <= kDynLds, "merge area");

struct Q2kArgs {
    const uint8_t* k_codes;     // [T/32][n_kv][D][8]
    const uint16_t* k_scale;    // [T/32][n_kv][D] fp16
    const uint8_t* v_blocks;    // [T][n_kv][D/32][18]
    const uint16_t* k_ovl;      // [n_sink + n_window + n_slack][n_kv][D] fp16
    const uint16_t* v_ovl;
    const float* q;             // [S][n_kv * G][D]
    float sm_scale;
    int64_t T;
    int32_t S;                  // query tokens (1: decode)
    int64_t pos0;               // token s attends cells t <= pos0 + s; < 0: every cell (decode)
    int32_t n_kv, n_sink, n_window;
    int32_t n_ring;             // window ring slots: n_window + n_slack
    int64_t ovl_a;              // first non-sink window cell, max(n_sink, T - n_window)
    int32_t ovl_ra;             // (ovl_a - n_sink) mod n_ring
    int32_t xcd_map;
    uint32_t lv_lo, lv_hi;      // low / high bytes of the 4 fp16 levels
    float lv_absmax;
    float* part_acc;            // [n_split][n_kv * G][D]
    float* part_ml;             // [n_split][n_kv * G][2]
};

__device__ __forceinline__ int headroom_exp(float x) {
    if (!(x > 0.0f)) return 0;
    int k;
    (void)frexpf(x, &k);
    return 14 - k;
}

__device__ __forceinline__ float f16v(uint32_t bits) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
__device__ __forceinline__ uint32_t pack2(_Float16 a, _Float16 b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// f32 x (already pre-scaled) -> f16 high part and f16 residual
__device__ __forceinline__ void split16(float x, _Float16& hi, _Float16& lo) {
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}

// overlay slot of cell t (or -1): a sink keeps slot t, a window cell its ring
// slot n_sink + (t - n_sink) mod n_ring, counted from the first window cell
// (t - ovl_a < n_window <= n_ring: one conditional subtraction, 32-bit)
__device__ __forceinline__ int64_t ovl_slot(int64_t t, const Q2kArgs& a) {
    if (t < a.n_sink) return t;
    if (t >= a.ovl_a) {
        int r = a.ovl_ra + (int)(t - a.ovl_a);
        r = r >= a.n_ring ? r - a.n_ring : r;
        return a.n_sink + r;
    }
    return -1;
}

// row of the 32-cell group held in context k slot e of lane group g
__device__ __forceinline__ int rho(int g, int e) { return 16 * (e >> 2) + 4 * g + (e & 3); }

struct GroupRegs {
    u32x4 kc[2];        // K codes of channels 4l..4l+3 (8 bytes each)
    u32x2 ks;           // their fp16 scales
    u32x4 v[5];         // 16-byte pieces lane, lane+64, ... of the group's V rows
};

__device__ __forceinline__ void load_group(GroupRegs& r, const Q2kArgs& a, int64_t grp, int kvh,
                                           int lane) {
    const int64_t gk = grp * a.n_kv + kvh;
    const uint8_t* kc = a.k_codes + (gk * D) * 8 + 32 * lane;
    r.kc[0] = *reinterpret_cast<const u32x4*>(kc);
    r.kc[1] = *reinterpret_cast<const u32x4*>(kc + 16);
    r.ks = *reinterpret_cast<const u32x2*>(a.k_scale + gk * D + 4 * lane);
    const int64_t cell0 = grp * CELLS;
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int p = lane + 64 * k;
        if (p < NPIECE) {
            const int cell = p / 9, piece = p % 9;
            r.v[k] = *reinterpret_cast<const u32x4*>(
                a.v_blocks + ((cell0 + cell) * a.n_kv + kvh) * RAWROW + 16 * piece);
        }
    }
}

// 4x4 byte transpose: out[q] byte k = in[k] byte q
__device__ __forceinline__ void transpose4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                           uint32_t (&o)[4]) {
    const uint32_t t0 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t t1 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    const uint32_t t2 = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
    const uint32_t t3 = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
    o[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);              // a0 b0 c0 d0
    o[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

__global__ __launch_bounds__(kThreads, 1) void k_q2k_mfma(Q2kArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float cf_s[kWaves][CELLS];   // per-cell K factor of overlay groups
    __shared__ float ml_s[kWaves][G][2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n16 = lane & 15;
    int b = blockIdx.x;
    if (a.xcd_map) b = (b & 7) * (gridDim.x >> 3) + (b >> 3);
    // block = (token, slice, KV head); slice `chunk` owns the groups chunk,
    // chunk + n_slices, ... below the token's causal limit
    const int per_tok = gridDim.x / a.S;
    const int tok = b / per_tok;
    const int chunk = (b % per_tok) / a.n_kv, kvh = b % a.n_kv;
    const int n_slices = per_tok / a.n_kv;
    const int64_t T = a.T;
    const int64_t lim = a.pos0 < 0 ? T : a.pos0 + tok + 1;   // cells this token attends
    const int64_t g_total = (lim + CELLS - 1) / CELLS;      // the last group may be partial
    const int n_groups = g_total > chunk ? (int)((g_total - chunk + n_slices - 1) / n_slices) : 0;
    auto grp_of = [&](int k) -> int64_t { return chunk + (int64_t)k * n_slices; };
    const int n_qrows = a.S * a.n_kv * G;
    const int64_t qrow0 = (int64_t)tok * a.n_kv * G + kvh * G;   // first query row of this block

    // ---- query: this lane's score B operand, head n16/2, its f16 high part
    // (n16 even) or residual (n16 odd) of q * 2^eq, channels 32s + 8g + [0, 8);
    // loaded before the first group, so it is ready first (loads return in
    // issue order).  The 4 lanes n16 + 16g hold the head's 256 channels.
    half8_t qb[KSTEPS];
    float hf;                               // score factor of the head (without the K pre-scale)
    GroupRegs pf;                           // this wave's next group, in flight
    {
        const float* src = a.q + (qrow0 + (n16 >> 1)) * D + 8 * g;
        float x[KSTEPS][8];
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
            const float4 u0 = *reinterpret_cast<const float4*>(src + 32 * s);
            const float4 u1 = *reinterpret_cast<const float4*>(src + 32 * s + 4);
            x[s][0] = u0.x; x[s][1] = u0.y; x[s][2] = u0.z; x[s][3] = u0.w;
            x[s][4] = u1.x; x[s][5] = u1.y; x[s][6] = u1.z; x[s][7] = u1.w;
        }
        if (wave < n_groups) load_group(pf, a, grp_of(wave), kvh, lane);
        float mx = 0.0f;
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(x[s][e]));
        mx = fmaxf(mx, xor_lane<16>(mx));
        mx = fmaxf(mx, xor_lane<32>(mx));
        const int eq = headroom_exp(mx);
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                _Float16 h, l;
                split16(ldexpf(x[s][e], eq), h, l);
                qb[s][e] = (n16 & 1) ? l : h;
            }
        hf = ldexpf(1.0f, -eq) * a.sm_scale * kLog2e;
    }

    uint8_t* base = lds + wave * WAVE_LDS;
    uint8_t* Bhi = base;                                // K hi, then V hi
    uint8_t* Blo = base + BUF;                          // K lo, then V lo
    uint8_t* raw = base + 2 * BUF;

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, m_used = -INFINITY, l_run = 0.0f;

    // V is staged as V * 2^ev_w: the first group with nonzero V sets ev_w from
    // its largest value (|V| <= 8 d for the bulk, the overlay values as they
    // are), and a later group with larger values lowers it, rescaling the
    // accumulator by the exact power of two
    int ev_w = 0;
    bool v_set = false;
    float d_mul = 1.0f;
    const int blk = lane & 7;                           // V block of this lane's (cell, block) pairs
    const bool blk_odd = (blk & 1) != 0;
    const half2_t m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};


    for (int gi = wave; gi < n_groups; gi += kWaves) {
        GroupRegs cur = pf;
        if (gi + kWaves < n_groups) load_group(pf, a, grp_of(gi + kWaves), kvh, lane);
        const int64_t cb = grp_of(gi) * CELLS;          // first cell of the group
        // cells attended (the causal limit, or the end of a cache built by
        // appends, may fall inside the group: cells past it stage bulk rows
        // with V zeroed and score -inf)
        const int n_here = (lim - cb < CELLS) ? (int)(lim - cb) : CELLS;
        const bool any_ovl = (cb < a.n_sink) || (cb + CELLS > T - a.n_window);
        const bool all_ovl = n_here == CELLS && ((cb + CELLS <= a.n_sink) || (cb >= T - a.n_window));

        // ---- 1. K hi/lo -> [cell][channel] ----
        // the group's bulk K is staged as K * 2^ek (largest level * scale of
        // the group in [2^13, 2^14)); its scores are scaled back by kbulk
        float mks = fmaxf(fmaxf(fabsf(f16v(cur.ks.x & 0xFFFFu)), fabsf(f16v(cur.ks.x >> 16))),
                          fmaxf(fabsf(f16v(cur.ks.y & 0xFFFFu)), fabsf(f16v(cur.ks.y >> 16))));
        mks = wave_max(mks);
        const int ek = headroom_exp(a.lv_absmax * mks);
        const float ks_mul = ldexpf(1.0f, ek), kbulk = ldexpf(1.0f, -ek);
        if (!all_ovl) {
            // scales of channels 4l..4l+3, pre-scaled (exact unless subnormal)
            const _Float16 s0 = (_Float16)(f16v(cur.ks.x & 0xFFFFu) * ks_mul);
            const _Float16 s1 = (_Float16)(f16v(cur.ks.x >> 16) * ks_mul);
            const _Float16 s2 = (_Float16)(f16v(cur.ks.y & 0xFFFFu) * ks_mul);
            const _Float16 s3 = (_Float16)(f16v(cur.ks.y >> 16) * ks_mul);
            const half2_t ks01 = {s0, s1}, ks23 = {s2, s3};
            uint32_t xq[8];
            {
                uint32_t t4[4];
                transpose4(cur.kc[0].x, cur.kc[0].z, cur.kc[1].x, cur.kc[1].z, t4);
                xq[0] = t4[0]; xq[1] = t4[1]; xq[2] = t4[2]; xq[3] = t4[3];
                transpose4(cur.kc[0].y, cur.kc[0].w, cur.kc[1].y, cur.kc[1].w, t4);
                xq[4] = t4[0]; xq[5] = t4[1]; xq[6] = t4[2]; xq[7] = t4[3];
            }
            uint8_t* dh = Bhi + 8 * lane;
            uint8_t* dl = Blo + 8 * lane;
#pragma unroll
            for (int qd = 0; qd < 8; ++qd) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int cell = 4 * qd + i;
                    const uint32_t codes = (xq[qd] >> (2 * i)) & 0x03030303u;
                    const uint32_t L = __builtin_amdgcn_perm(a.lv_hi, a.lv_lo, codes);
                    const uint32_t H = __builtin_amdgcn_perm(a.lv_hi, a.lv_lo, codes | 0x04040404u);
                    const half2_t v01 = as_h2(__builtin_amdgcn_perm(H, L, 0x05010400u));
                    const half2_t v23 = as_h2(__builtin_amdgcn_perm(H, L, 0x07030602u));
                    const half2_t h01 = v01 * ks01, h23 = v23 * ks23;
                    const half2_t l01 = __builtin_elementwise_fma(v01, ks01, -h01);
                    const half2_t l23 = __builtin_elementwise_fma(v23, ks23, -h23);
                    *reinterpret_cast<u32x2*>(dh + cell * ROW) = u32x2{as_u(h01), as_u(h23)};
                    *reinterpret_cast<u32x2*>(dl + cell * ROW) = u32x2{as_u(l01), as_u(l23)};
                }
            }
        }
        // overlay cells of the group: lane (cell lane/2, channel half lane%2)
        // reads its 256 bytes of the fp16 copy with 16-byte loads
        const int ocl = lane >> 1, ohf = lane & 1;
        const int64_t oslot = (any_ovl && ocl < n_here) ? ovl_slot(cb + ocl, a) : -1;
        const bool oov = oslot >= 0;
        const int64_t ooff = ((oov ? oslot : 0) * a.n_kv + kvh) * D + 128 * ohf;   // elements
        uint8_t* const orow_h = Bhi + ocl * ROW + 256 * ohf;
        uint8_t* const orow_l = Blo + ocl * ROW + 256 * ohf;
        if (any_ovl) {
            // the fp16 copies are exact f16 operands: residual 0, score factor 1
            u32x4 ko[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) ko[u] = *reinterpret_cast<const u32x4*>(a.k_ovl + ooff + 8 * u);
            if (oov) {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    *reinterpret_cast<u32x4*>(orow_h + 16 * u) = ko[u];
                    *reinterpret_cast<u32x4*>(orow_l + 16 * u) = u32x4{0u, 0u, 0u, 0u};
                }
            }
            if (ohf == 0) cf_s[wave][ocl] = oov ? 1.0f : kbulk;
        }
        // ---- 2. scores: cells 16t + n16 (A rows) x query columns n16 ----
        f32x4 sc4[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
            const uint8_t* ph = Bhi + (16 * t + n16) * ROW + 16 * g;
            const uint8_t* pl = Blo + (16 * t + n16) * ROW + 16 * g;
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const half8_t Ah = *reinterpret_cast<const half8_t*>(ph + 64 * ks);
                const half8_t Al = *reinterpret_cast<const half8_t*>(pl + 64 * ks);
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, qb[ks], s, 0, 0, 0);
                s = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, qb[ks], s, 0, 0, 0);
            }
            sc4[t] = s;
        }

        // ---- 3. online softmax over the group's 32 cells (rows rho(g, e)) ----
        float sc[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = sc4[t][i];
                sc[4 * t + i] = v + xor_lane<1>(v);   // high-part column + residual column
            }
        if (any_ovl) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] *= hf * cf_s[wave][rho(g, e)];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[e] *= hf * kbulk;
        }
        if (n_here < CELLS) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (rho(g, e) >= n_here) sc[e] = -INFINITY;
        }
        float tmax = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
        tmax = fmaxf(tmax, xor_lane<16>(tmax));
        tmax = fmaxf(tmax, xor_lane<32>(tmax));
        m_run = fmaxf(m_run, tmax);
        const bool need = m_run > m_used + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(need) != 0ull) {
            const float m_new = need ? m_run : m_used;
            const float alpha = (m_used == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_used - m_new);
            l_run *= alpha;
            m_used = m_new;
            // accumulator row 4g + i belongs to head (4g + i) / 2, whose state
            // lane 4g + 2*(i/2) holds
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * g + 2 * (i >> 1));
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t][i] *= ai;
            }
        }
        half8_t pa;                                     // A operand: row n16 = (head, part)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(sc[e] - m_used);
            l_run += p;
            _Float16 h, l;
            split16(p * kPScale, h, l);
            pa[e] = (n16 & 1) ? l : h;
        }

        // ---- 4. V hi/lo -> [cell][channel] (same LDS, after the K reads) ----
        u32x4 vo[16];
        if (any_ovl) {
#pragma unroll
            for (int u = 0; u < 16; ++u) vo[u] = *reinterpret_cast<const u32x4*>(a.v_ovl + ooff + 8 * u);
        }
        // largest staged magnitude of the group: 8 d over the bulk blocks, the
        // overlay values as they are
        float vneed = 0.0f;
        uint32_t wv[4][5];                              // this lane's 4 (cell, block) pairs, raw words
        if (!all_ovl) {
#pragma unroll
            for (int k = 0; k < 5; ++k) {
                const int p = lane + 64 * k;
                if (p < NPIECE) *reinterpret_cast<u32x4*>(raw + (p / 9) * RAWROW + 16 * (p % 9)) = cur.v[k];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int cell = (lane + 64 * k) >> 3;
                const uint32_t* rw = reinterpret_cast<const uint32_t*>(raw + cell * RAWROW + ((18 * blk) & ~3));
#pragma unroll
                for (int i = 0; i < 5; ++i) wv[k][i] = rw[i];
            }
            if (n_here < CELLS) {                       // cells past the limit: d = 0, values 0
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (((lane + 64 * k) >> 3) >= n_here)
#pragma unroll
                        for (int i = 0; i < 5; ++i) wv[k][i] = 0u;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t dbits = blk_odd ? (wv[k][0] >> 16) : (wv[k][0] & 0xFFFFu);
                vneed = fmaxf(vneed, 8.0f * fabsf(f16v(dbits)));
            }
        }
        if (any_ovl && oov) {
            half2_t m2 = {(_Float16)0.0f, (_Float16)0.0f};
#pragma unroll
            for (int u = 0; u < 16; ++u)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    m2 = __builtin_elementwise_max(m2, __builtin_elementwise_abs(as_h2(vo[u][c])));
            vneed = fmaxf(vneed, fmaxf((float)m2[0], (float)m2[1]));
        }
        const float vmx = wave_max(vneed);
        if (vmx > 0.0f) {
            const int e_need = headroom_exp(vmx);
            if (!v_set) {                               // nothing accumulated yet
                ev_w = e_need;
                v_set = true;
            } else if (e_need < ev_w) {
                const float r = ldexpf(1.0f, e_need - ev_w);
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[t] *= r;
                ev_w = e_need;
            }
            d_mul = ldexpf(1.0f, ev_w);
        }
        if (!all_ovl) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int cell = (lane + 64 * k) >> 3;
                const uint32_t* w = wv[k];
                const uint32_t dbits = blk_odd ? (w[0] >> 16) : (w[0] & 0xFFFFu);
                const _Float16 dsc = (_Float16)(f16v(dbits) * d_mul);
                const half2_t dd = {dsc, dsc};
                uint32_t lo_o[8], hi_o[8], lo_h[8], hi_h[8];   // [low-nibble | high-nibble] x [hi | lo]
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t n = blk_odd ? w[i + 1] : __builtin_amdgcn_alignbyte(w[i + 1], w[i], 2);
                    const uint32_t nl = n & 0x0F0F0F0Fu, nh = (n >> 4) & 0x0F0F0F0Fu;
                    const half2_t a0 = as_h2(__builtin_amdgcn_perm(0x64646464u, nl, 0x04010400u)) + m1032;
                    const half2_t a1 = as_h2(__builtin_amdgcn_perm(0x64646464u, nl, 0x04030402u)) + m1032;
                    const half2_t b0 = as_h2(__builtin_amdgcn_perm(0x64646464u, nh, 0x04010400u)) + m1032;
                    const half2_t b1 = as_h2(__builtin_amdgcn_perm(0x64646464u, nh, 0x04030402u)) + m1032;
                    const half2_t ha0 = a0 * dd, ha1 = a1 * dd, hb0 = b0 * dd, hb1 = b1 * dd;
                    hi_o[2 * i] = as_u(ha0);
                    hi_o[2 * i + 1] = as_u(ha1);
                    hi_h[2 * i] = as_u(hb0);
                    hi_h[2 * i + 1] = as_u(hb1);
                    lo_o[2 * i] = as_u(__builtin_elementwise_fma(a0, dd, -ha0));
                    lo_o[2 * i + 1] = as_u(__builtin_elementwise_fma(a1, dd, -ha1));
                    lo_h[2 * i] = as_u(__builtin_elementwise_fma(b0, dd, -hb0));
                    lo_h[2 * i + 1] = as_u(__builtin_elementwise_fma(b1, dd, -hb1));
                }
                // channels 32*blk + 0..15 (low nibbles) and 32*blk + 16..31 (high nibbles)
                uint8_t* rh = Bhi + cell * ROW + 64 * blk;
                uint8_t* rl = Blo + cell * ROW + 64 * blk;
                *reinterpret_cast<u32x4*>(rh) = u32x4{hi_o[0], hi_o[1], hi_o[2], hi_o[3]};
                *reinterpret_cast<u32x4*>(rh + 16) = u32x4{hi_o[4], hi_o[5], hi_o[6], hi_o[7]};
                *reinterpret_cast<u32x4*>(rh + 32) = u32x4{hi_h[0], hi_h[1], hi_h[2], hi_h[3]};
                *reinterpret_cast<u32x4*>(rh + 48) = u32x4{hi_h[4], hi_h[5], hi_h[6], hi_h[7]};
                *reinterpret_cast<u32x4*>(rl) = u32x4{lo_o[0], lo_o[1], lo_o[2], lo_o[3]};
                *reinterpret_cast<u32x4*>(rl + 16) = u32x4{lo_o[4], lo_o[5], lo_o[6], lo_o[7]};
                *reinterpret_cast<u32x4*>(rl + 32) = u32x4{lo_h[0], lo_h[1], lo_h[2], lo_h[3]};
                *reinterpret_cast<u32x4*>(rl + 48) = u32x4{lo_h[4], lo_h[5], lo_h[6], lo_h[7]};
            }
        }
        if (any_ovl && oov) {
            // fp16 copy * 2^ev_w as f16 high + residual: packed f16 when the
            // scale is an f16 normal (the product of an f16 and a power of two
            // rounds once, the fma gives the exact residual), else through f32
            if (ev_w >= -14 && ev_w <= 15) {
                const _Float16 sc16 = (_Float16)d_mul;
                const half2_t s2 = {sc16, sc16};
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    u32x4 h, l;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const half2_t x2 = as_h2(vo[u][c]);
                        const half2_t hh = x2 * s2;
                        h[c] = as_u(hh);
                        l[c] = as_u(__builtin_elementwise_fma(x2, s2, -hh));
                    }
                    *reinterpret_cast<u32x4*>(orow_h + 16 * u) = h;
                    *reinterpret_cast<u32x4*>(orow_l + 16 * u) = l;
                }
            } else {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    u32x4 h, l;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        _Float16 h0, l0, h1, l1;
                        split16(f16v(vo[u][c] & 0xFFFFu) * d_mul, h0, l0);
                        split16(f16v(vo[u][c] >> 16) * d_mul, h1, l1);
                        h[c] = pack2(h0, h1);
                        l[c] = pack2(l0, l1);
                    }
                    *reinterpret_cast<u32x4*>(orow_h + 16 * u) = h;
                    *reinterpret_cast<u32x4*>(orow_l + 16 * u) = l;
                }
            }
        }

        // ---- 5. context: V operand rows rho(g, 0..3) and rho(g, 4..7), column n16 ----
        {
            const int src_row = 4 * g + (n16 >> 2);
            const uint8_t* vh0 = Bhi + src_row * ROW + 8 * (n16 & 3);
            const uint8_t* vl0 = Blo + src_row * ROW + 8 * (n16 & 3);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(vh0 + 32 * t));
                const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(vh0 + 16 * ROW + 32 * t));
                const i16x4 l0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(vl0 + 32 * t));
                const i16x4 l1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(vl0 + 16 * ROW + 32 * t));
                const half8_t Bh = __builtin_shufflevector(__builtin_bit_cast(half4_t, h0),
                                                           __builtin_bit_cast(half4_t, h1),
                                                           0, 1, 2, 3, 4, 5, 6, 7);
                const half8_t Bl = __builtin_shufflevector(__builtin_bit_cast(half4_t, l0),
                                                           __builtin_bit_cast(half4_t, l1),
                                                           0, 1, 2, 3, 4, 5, 6, 7);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, Bh, acc[t], 0, 0, 0);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, Bl, acc[t], 0, 0, 0);
            }
        }
    }

    // ---- merge the 4 waves in LDS, add the two rows of each head, write the partial ----
    l_run += xor_lane<16>(l_run);
    l_run += xor_lane<32>(l_run);
    __syncthreads();                                    // staging areas consumed
    if (g == 0 && (n16 & 1) == 0) {
        ml_s[wave][n16 >> 1][0] = m_used;
        ml_s[wave][n16 >> 1][1] = l_run;
    }
    __syncthreads();
    float* red = reinterpret_cast<float*>(lds);        // [wave][16 rows][D]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i, h = row >> 1;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml_s[w][h][0]);
        const float mw = ml_s[wave][h][0];
        const float f = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M) * ldexpf(1.0f, -ev_w);
        float* dst = red + (wave * 16 + row) * D + n16;
#pragma unroll
        for (int t = 0; t < NT; ++t) dst[16 * t] = acc[t][i] * f;
    }
    __syncthreads();
    const float unscale = 1.0f / kPScale;
    for (int idx = tid; idx < G * D / 4; idx += kThreads) {
        const int h = idx / (D / 4), dd = 4 * (idx % (D / 4));
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            s += *reinterpret_cast<const f32x4*>(red + (w * 16 + 2 * h) * D + dd);
            s += *reinterpret_cast<const f32x4*>(red + (w * 16 + 2 * h + 1) * D + dd);
        }
        // read once, by the combine pass: streaming stores
        __builtin_nontemporal_store(s * unscale, reinterpret_cast<f32x4*>(
                                                     a.part_acc + ((int64_t)chunk * n_qrows + qrow0 + h) * D + dd));
    }
    if (tid < G) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, ml_s[w][tid][0]);
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = ml_s[w][tid][0];
            L += (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M) * ml_s[w][tid][1];
        }
        float* ml = a.part_ml + ((int64_t)chunk * n_qrows + qrow0 + tid) * 2;
        ml[0] = M;
        ml[1] = L;
    }
}

}  // namespace

bool q2k_mfma_eligible(const kvq_cache& kv, int32_t Hq, int32_t S, const void* q) {
    auto al = [](const void* p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
    const bool ovl = (kv.n_sink + kv.n_window) > 0;
    return kv.fmt == KVQ_Q2K && kv.d == D && S >= 1 && (int64_t)S * kv.n_kv <= (1 << 16) &&
           kv.n_kv >= 1 && Hq == G * kv.n_kv &&
           al(kv.codes, 16) && al(kv.scales, 8) &&
           al(kv.v_blocks, 16) && al(q, 16) && (!ovl || (al(kv.k_ovl, 16) && al(kv.v_ovl, 16)));
}

// about one workgroup per CU: ~256 / n_kv slices of the 32-cell groups
void q2k_mfma_plan(const kvq_cache& kv, int32_t Hq, int32_t S, AttnPlan& p) {
    const int64_t groups = (kv.n_rows + CELLS - 1) / CELLS;
    int64_t want = (256 + (int64_t)kv.n_kv * S - 1) / ((int64_t)kv.n_kv * S);
    if (want > groups) want = groups;
    if (want < 1) want = 1;
    p.path = 2;
    p.n_split = (int32_t)want;
    p.chunk = ((groups + want - 1) / want) * CELLS;      // cells per slice (at most)
    p.n_qrows = Hq * S;
    p.heads_per_blk = G;
    p.n_qgroups = kv.n_kv * S;
    p.log2_domain = 1;
    p.ws_bytes = (size_t)p.n_split * p.n_qrows * (D + 2) * sizeof(float);
}

hipError_t launch_q2k_mfma(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                           int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                           float* part_ml, hipStream_t s) {
    (void)Hq;
    Q2kArgs a;
    a.k_codes = kv.codes;
    a.k_scale = reinterpret_cast<const uint16_t*>(kv.scales);
    a.v_blocks = kv.v_blocks;
    a.k_ovl = kv.k_ovl;
    a.v_ovl = kv.v_ovl;
    a.q = q;
    a.sm_scale = sm_scale;
    a.T = kv.n_rows;
    a.S = S;
    a.pos0 = S == 1 && pos0 < 0 ? -1 : pos0;
    a.n_kv = kv.n_kv;
    a.n_sink = kv.n_sink;
    a.n_window = kv.n_window;
    a.n_ring = kv.n_window + kv.n_slack;
    {
        const int64_t wb = kv.n_rows - kv.n_window;
        a.ovl_a = wb > kv.n_sink ? wb : kv.n_sink;
        a.ovl_ra = a.n_ring > 0 ? (int32_t)((a.ovl_a - kv.n_sink) % a.n_ring) : 0;
    }
    const int blocks = p.n_split * kv.n_kv * S;
    a.xcd_map = (blocks % 8 == 0) ? 1 : 0;
    const Codebook4& cb = codebook4();
    uint32_t lo = 0, hi = 0;
    float amax = 0.0f;
    for (int i = 0; i < 4; ++i) {
        const _Float16 h = (_Float16)cb.level[i];
        const uint16_t bits = __builtin_bit_cast(uint16_t, h);
        lo |= (uint32_t)(bits & 0xFFu) << (8 * i);
        hi |= (uint32_t)(bits >> 8) << (8 * i);
        amax = fmaxf(amax, fabsf(cb.level[i]));
    }
    a.lv_lo = lo;
    a.lv_hi = hi;
    a.lv_absmax = amax;
    a.part_acc = part_acc;
    a.part_ml = part_ml;
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_dyn_lds_once(reinterpret_cast<const void*>(&k_q2k_mfma), kDynLds, lds_set);
    if (e != hipSuccess) return e;
    k_q2k_mfma<<<blocks, kThreads, kDynLds, s>>>(a);
    return hipGetLastError();
}

}  // namespace kvq
