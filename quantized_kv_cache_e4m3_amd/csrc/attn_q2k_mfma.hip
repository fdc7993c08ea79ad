// GQA decode attention over a q2k cache (d = 256 per KV head, 8 query heads
// per KV head) on the gfx950 matrix cores, and its combine step.
//
// [Strata #2318] "Summary" items 1-3 and "Why per-channel K and per-token V":
// bulk K is a 2-bit level per (cell, channel) times an fp16 scale per
// (32-cell group, channel); bulk V is q4_0, (code - 8) times an fp16 scale
// per (cell, 32-channel block); the first n_sink cells and the last n_window
// cells read exact fp16 copies instead.  The cache is read as stored.
//
// Split of the work.  The decode kernel attends the bulk cells (the cells
// between the sinks and the window).  For one decode token whose bulk groups
// leave enough waves free (each slice's waves take one group each, and the
// window's 32-cell groups fit the waves left over: at T = 32768 with 2 KV
// heads, 1016 bulk groups and 8 window groups fill the 1024 waves per KV head
// exactly), those waves attend the window from its exact fp16 ring rows on
// the same matrix cores, so it costs the launch no time.  The remaining
// overlay cells (the sinks, or the whole overlay when the window does not fit
// the free waves) are attended in f32 by the combine kernel, which reads
// their fp16 copies directly and merges them with the decode kernel's chunk
// partials.
//
// Decode: both products are MFMA v_mfma_f32_16x16x32_f16 with exact f16
// operands:
//   scores   S[cell, 2h+p] = sum_c K[cell, c] * Qp[h][c]      (p: query hi/lo)
//   context  C[2h+p, c]   += sum_cell Pp[h][cell] * V[cell, c] (p: weight hi/lo)
// The 8 query heads fill the 16 MFMA columns (rows) twice: once with the f16
// high part of the pre-scaled query (weight), once with its f16 residual, so
// one MFMA carries both terms of the split.  K = level * scale and
// V = (code - 8) * d have up to 22 and 15 significant bits, so each is formed
// in registers as an exact f16 pair hi + lo (v_pk_mul_f16 for hi, v_pk_fma_f16
// for the exact residual) and multiplied twice.  The scales carry
// power-of-two pre-scales chosen from the stored values so that nothing
// overflows f16: one per group for K (its scores are scaled back), one per
// wave for V, set by the wave's first group and lowered (rescaling the
// accumulator by the exact power of two) when a later group holds larger
// values.
//
// Operands straight from the stored bits.  Per group a wave copies the K
// codes as stored ([channel][8 bytes], 32 cells of 2 bits) into its LDS area,
// and the V nibbles realigned to 16 bytes per (cell, block), rows in the
// context's k order.  ds_read_b64_tr_b8 then hands every lane its operand
// bytes: for the score A operand, byte i of 8 channel words holds cells
// 4i .. 4i+3 of those 8 channels, so lane (n16, g) takes channels
// 32s + 8g + [0, 8) of cell 4 (n16 % 8) + 2t + n16 / 8 in tile t (the two
// tiles share one read); for the V operand, byte n16 of a block's nibble row
// holds channels n16 and n16 + 16 of 8 cells (two tiles per read).  The
// levels come from a 4-entry byte table (v_perm), the nibbles become f16
// through the 0x6400 exponent trick.  Row (t, r) of the score tiles is cell
// 4 (r % 8) + 2t + r / 8, and the score MFMA's output element (t, i) of lane
// (n16, g) is then the context's k position 8g + 4t + i.
//
// Work layout.  Workgroup = (slice of 32-cell groups, KV head), 8 waves (two
// per SIMD); slice j of n holds the bulk groups j, j + n, j + 2n, ...; wave w
// takes the slice's groups w, w + 8, ... with a private online softmax and
// private accumulators, merged in LDS at the end into one (m, l, acc) partial
// per slice (m in log2 units).
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int D = 256;                  // channels per KV head
constexpr int G = 8;                    // query heads per KV head
constexpr int CELLS = 32;               // cells per group
constexpr int NBLK = D / 32;            // q4_0 blocks per cell
constexpr int KSTEPS = D / 32;          // score k-steps
constexpr int NT = D / 16;              // context dim tiles
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int VROW = NBLK * 18;         // bytes of one cell's V blocks for one KV head
// per-wave LDS area
constexpr int KC_OFF = 0;                       // K codes as stored: [256 channels][8 bytes]
constexpr int SC_OFF = KC_OFF + D * 8;          // pre-scaled K scales, f16 [256]
constexpr int NBR = 128 + 16;                   // nibble row stride (16 bytes of padding)
constexpr int NB_OFF = SC_OFF + D * 2;          // V nibbles [32 k positions][NBR]
constexpr int DV_OFF = NB_OFF + CELLS * NBR;    // pre-scaled V scales, f16 [8 blocks][32 k positions]
constexpr int RAW_OFF = DV_OFF + NBLK * CELLS * 2;   // the group's V rows as stored [32 cells][144 B]
constexpr int BULK_LDS = RAW_OFF + CELLS * VROW;
// a window group's value rows, f16 [32 cells][256 channels], rows padded by
// 16 bytes (the transpose reads stay bank-conflict free)
constexpr int WLDR = 2 * D + 16;
constexpr int WIN_LDS = CELLS * WLDR;
constexpr int WAVE_LDS = BULK_LDS > WIN_LDS ? BULK_LDS : WIN_LDS;
constexpr int NPIECE = CELLS * VROW / 16;       // 288 16-byte pieces of a group's V rows
constexpr int kMergeLds = kWaves * 16 * D * 4;  // accumulators of the 8 waves
constexpr int kDynLds = kMergeLds > kWaves * WAVE_LDS ? kMergeLds : kWaves * WAVE_LDS;
constexpr float kRescaleSlack = 1.0f;   // log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPScale = 4096.0f;      // weights p <= 2 staged as p * 2^12 (< 2^14)
constexpr int kBufWord3 = 0x00020000;   // gfx9 buffer descriptor word 3 (32-bit data format)

static_assert(kDynLds <= 160 * 1024 - 1024, "LDS budget");

struct Q2kArgs {
    const uint8_t* k_codes;     // [T/32][n_kv][D][8]
    const uint16_t* k_scale;    // [T/32][n_kv][D] fp16
    const uint8_t* v_blocks;    // [T][n_kv][D/32][18]
    const float* q;             // [S][n_kv * G][D]
    float sm_scale;
    int64_t T;
    int32_t S;                  // query tokens (1: decode)
    int64_t pos0;               // token s attends cells t <= pos0 + s; < 0: every cell (decode)
    int32_t n_kv;
    int64_t bulk_lo, bulk_hi;   // cells [bulk_lo, bulk_hi) are read from the bulk codes
    int32_t xcd_map;
    uint32_t lv_lo, lv_hi;      // low / high bytes of the 4 fp16 levels
    float lv_absmax;
    float* part_acc;            // [n_split][S * n_kv * G][D]
    float* part_ml;             // [n_split][S * n_kv * G][2]
    // window cells attended here (win_groups > 0: one decode token whose bulk
    // groups leave a wave free in every slice position the window needs)
    const uint16_t* k_ovl;      // [n_ovl][n_kv][D] fp16
    const uint16_t* v_ovl;
    int32_t ovl_bytes;          // bytes of either overlay array
    int32_t n_sink;
    int32_t ovl_ra, n_ring;     // ring slot of the first window cell, ring length
    int32_t n_win;              // window cells (all attended: decode)
    int32_t win_groups;         // ceil(n_win / 32), 0: the combine attends the window
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

// f32 x (already pre-scaled) -> f16 high part and f16 residual
__device__ __forceinline__ void split16(float x, _Float16& hi, _Float16& lo) {
    hi = (_Float16)x;
    lo = (_Float16)(x - (float)hi);
}

// k position (context k index) of the group's cell c: the score tile row of
// c is (t, r) with r % 8 = c / 4, t = (c % 4) / 2, r / 8 = c % 2, and the
// score output element (t, i) of lane group g is position 8g + 4t + i with
// r = 4g + i
__device__ __forceinline__ int kpos(int c) {
    const int sub = c & 3;
    return 16 * (sub & 1) + 8 * (c >> 4) + 4 * (sub >> 1) + ((c >> 2) & 3);
}
// cell at output element (t, i) of lane group g (the inverse of kpos)
__device__ __forceinline__ int cell_at(int g, int t, int i) {
    const int r = 4 * g + i;
    return 4 * (r & 7) + 2 * t + (r >> 3);
}

// one group's bulk data for this lane, in flight
struct GroupRegs {
    u32x4 kc0, kc1;     // K codes of channels 4l .. 4l+3 (8 bytes each)
    u32x2 ks;           // their fp16 scales
    u32x4 v[5];         // V rows: 16-byte pieces l, l + 64, ... (cell p / 9, piece p % 9)
};

// Loads of group grp (valid = false: none of its data, every load reads 0).
// Range-checked buffer loads with no branch, so the counter waits that follow
// know exactly which loads are in flight.
__device__ __forceinline__ void load_group(GroupRegs& r, const Q2kArgs& a, int64_t grp, bool valid,
                                           int kvh, int lane) {
    const int64_t gk = grp * a.n_kv + kvh;
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.k_codes + gk * (D * 8)), (short)0, valid ? D * 8 : 0, kBufWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.k_scale + gk * D), (short)0, valid ? D * 2 : 0, kBufWord3);
    r.kc0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, 32 * lane, 0, 0));
    r.kc1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, 32 * lane + 16, 0, 0));
    r.ks = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(sr, 8 * lane, 0, 0));
    // the group's V rows present in the cache (cells past T read 0)
    const int64_t cb = grp * CELLS;
    const int n_cells = !valid ? 0 : (a.T - cb < CELLS) ? (int)(a.T - cb) : CELLS;
    const int rowb = a.n_kv * VROW;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.v_blocks + cb * rowb), (short)0, n_cells * rowb, kBufWord3);
#pragma unroll
    for (int k = 0; k < 5; ++k) {
        const int p = lane + 64 * k;            // pieces past the group's 288 read 0
        r.v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                               rs, p < NPIECE ? (p / 9) * rowb + kvh * VROW + 16 * (p % 9)
                                                              : CELLS * rowb, 0, 0));
    }
}

__device__ __forceinline__ uint32_t align2(uint32_t hi, uint32_t lo) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// 8 codes (byte e of c0 / c1 = channel e / 4 + e of the k-step, values 0..3)
// -> their 8 f16 levels
__device__ __forceinline__ half8_t levels8(uint32_t c0, uint32_t c1, uint32_t lv_lo, uint32_t lv_hi) {
    const uint32_t l0 = __builtin_amdgcn_perm(lv_hi, lv_lo, c0);
    const uint32_t h0 = __builtin_amdgcn_perm(lv_hi, lv_lo, c0 | 0x04040404u);
    const uint32_t l1 = __builtin_amdgcn_perm(lv_hi, lv_lo, c1);
    const uint32_t h1 = __builtin_amdgcn_perm(lv_hi, lv_lo, c1 | 0x04040404u);
    const u32x4 w = {__builtin_amdgcn_perm(h0, l0, 0x05010400u), __builtin_amdgcn_perm(h0, l0, 0x07030602u),
                     __builtin_amdgcn_perm(h1, l1, 0x05010400u), __builtin_amdgcn_perm(h1, l1, 0x07030602u)};
    return __builtin_bit_cast(half8_t, w);
}

// 8 nibbles (low 4 bits of each byte of n0 / n1) -> f16 (nibble - 8), exact
__device__ __forceinline__ half8_t nib8(uint32_t n0, uint32_t n1) {
    const u32x4 w = {__builtin_amdgcn_perm(0x64646464u, n0, 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, n0, 0x04030402u),
                     __builtin_amdgcn_perm(0x64646464u, n1, 0x04010400u),
                     __builtin_amdgcn_perm(0x64646464u, n1, 0x04030402u)};
    const half8_t m1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f,
                           (_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f, (_Float16)-1032.0f};
    return __builtin_bit_cast(half8_t, w) + m1032;
}

__global__ __launch_bounds__(kThreads, 1) void k_q2k_mfma(Q2kArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float ml_s[kWaves][G][2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n16 = lane & 15;
    int b = blockIdx.x;
    if (a.xcd_map) b = (b & 7) * (gridDim.x >> 3) + (b >> 3);
    // block = (token, slice, KV head); slice `chunk` owns the bulk groups
    // g_first + chunk, g_first + chunk + n_slices, ... below the token's limit
    const int per_tok = gridDim.x / a.S;
    const int tok = b / per_tok;
    const int chunk = (b % per_tok) / a.n_kv, kvh = b % a.n_kv;
    const int n_slices = per_tok / a.n_kv;
    const int64_t lim = a.pos0 < 0 ? a.T : a.pos0 + tok + 1;   // cells this token attends
    const int64_t c_lo = a.bulk_lo;
    const int64_t c_hi = lim < a.bulk_hi ? lim : a.bulk_hi;    // bulk cells [c_lo, c_hi)
    const int64_t g_first = c_lo / CELLS;
    const int64_t n_grp = c_hi > c_lo ? (c_hi + CELLS - 1) / CELLS - g_first : 0;
    const int n_groups = n_grp > chunk ? (int)((n_grp - chunk + n_slices - 1) / n_slices) : 0;
    auto grp_of = [&](int k) -> int64_t { return g_first + chunk + (int64_t)k * n_slices; };
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
        load_group(pf, a, wave < n_groups ? grp_of(wave) : g_first, wave < n_groups, kvh, lane);
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

    uint8_t* const area = lds + wave * WAVE_LDS;
    // per-lane LDS addresses of the transposed operand reads and their scales
    const uint8_t* const kc_rd = area + KC_OFF + (8 * g + (n16 >> 1)) * 8;
    const uint8_t* const sc_rd = area + SC_OFF + 16 * g;
    const uint8_t* const nb_rd = area + NB_OFF + (8 * g + (n16 >> 1)) * NBR + 8 * (n16 & 1);
    const uint8_t* const dv_rd = area + DV_OFF + 16 * g;
    const int hsub = 2 * (n16 >> 3);        // bit offset of this lane's cell in a code byte (tile 0)

    f32x4 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, m_used = -INFINITY, l_run = 0.0f;

    // V is taken as V * 2^ev_w: the first group with nonzero V sets ev_w from
    // its largest value (|V| <= 8 d), and a later group with larger values
    // lowers it, rescaling the accumulator by the exact power of two
    int ev_w = 0;
    bool v_set = false;
    float d_mul = 1.0f;
    const int blk = lane & 7;               // V block of this lane's (cell, block) pairs
    const bool blk_odd = (blk & 1) != 0;

    // online softmax step over a group's 8 scores per lane (k positions
    // 8g + e, -inf for cells not attended): running max with lazy rescale,
    // then the weights p * 2^12 as the context's A operand (f16 high part in
    // the even rows, residual in the odd rows)
    auto weights = [&](const float (&sc)[8]) -> half8_t {
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
        half8_t w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(sc[e] - m_used);
            l_run += p;
            _Float16 h, l;
            split16(p * kPScale, h, l);
            w[e] = (n16 & 1) ? l : h;
        }
        return w;
    };

    for (int gi = wave; gi < n_groups; gi += kWaves) {
        const int64_t cb = grp_of(gi) * CELLS;         // first cell of the group
        // bulk cells of the group this token attends: [lo_c, hi_c)
        const int lo_c = (c_lo > cb) ? (int)(c_lo - cb) : 0;
        const int hi_c = (c_hi - cb < CELLS) ? (int)(c_hi - cb) : CELLS;

        // ---- stage the group: K codes as stored, pre-scaled K scales ----
        *reinterpret_cast<u32x4*>(area + KC_OFF + 32 * lane) = pf.kc0;
        *reinterpret_cast<u32x4*>(area + KC_OFF + 32 * lane + 16) = pf.kc1;
        // K taken as K * 2^ek: largest level * scale of the group in [2^13, 2^14)
        float mks = fmaxf(fmaxf(fabsf(f16v(pf.ks.x & 0xFFFFu)), fabsf(f16v(pf.ks.x >> 16))),
                          fmaxf(fabsf(f16v(pf.ks.y & 0xFFFFu)), fabsf(f16v(pf.ks.y >> 16))));
        mks = wave_max(mks);
        const int ek = headroom_exp(a.lv_absmax * mks);
        const float ks_mul = ldexpf(1.0f, ek), kbulk = ldexpf(1.0f, -ek);
        *reinterpret_cast<u32x2*>(area + SC_OFF + 8 * lane) =
            u32x2{pack2((_Float16)(f16v(pf.ks.x & 0xFFFFu) * ks_mul), (_Float16)(f16v(pf.ks.x >> 16) * ks_mul)),
                  pack2((_Float16)(f16v(pf.ks.y & 0xFFFFu) * ks_mul), (_Float16)(f16v(pf.ks.y >> 16) * ks_mul))};
        // ---- scores: tile t row r = cell 4 (r % 8) + 2t + r / 8 ----
        f32x4 sc4[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const i32x2 kb = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (i32x2 __attribute__((address_space(3)))*)(kc_rd + 256 * ks));
            const half8_t sp = *reinterpret_cast<const half8_t*>(sc_rd + 64 * ks);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int sh = 4 * t + hsub;
                const half8_t lv = levels8(((uint32_t)kb.x >> sh) & 0x03030303u,
                                           ((uint32_t)kb.y >> sh) & 0x03030303u, a.lv_lo, a.lv_hi);
                const half8_t kh = lv * sp;
                const half8_t kl = __builtin_elementwise_fma(lv, sp, -kh);
                sc4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, qb[ks], sc4[t], 0, 0, 0);
                sc4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kl, qb[ks], sc4[t], 0, 0, 0);
            }
        }

        // ---- online softmax over the group's cells (k positions 8g + e) ----
        float sc[8];
        const float fs = hf * kbulk;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = sc4[t][i];
                sc[4 * t + i] = (v + xor_lane<1>(v)) * fs;   // high-part column + residual column
            }
        if (lo_c > 0 || hi_c < CELLS) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = cell_at(g, e >> 2, e & 3);
                if (c < lo_c || c >= hi_c) sc[e] = -INFINITY;
            }
        }
        const half8_t pa = weights(sc);                 // A operand: row n16 = (head, part)

        // V rows as stored, then the nibbles realigned to 16 bytes per block
        // (rows in k order); the block scales of cells outside [lo_c, hi_c) are 0
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const int p = lane + 64 * k;
            if (p < NPIECE) *reinterpret_cast<u32x4*>(area + RAW_OFF + 16 * p) = pf.v[k];
        }
        // the next group's loads (after this group's registers are consumed)
        if (gi + kWaves < n_groups) load_group(pf, a, grp_of(gi + kWaves), true, kvh, lane);
        float vneed = 0.0f;
        uint32_t dbits[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int cell = (lane >> 3) + 8 * k;
            const uint32_t* rw = reinterpret_cast<const uint32_t*>(area + RAW_OFF + cell * VROW + ((18 * blk) & ~3));
            uint32_t w[5];
#pragma unroll
            for (int i = 0; i < 5; ++i) w[i] = rw[i];
            const u32x4 nib = blk_odd ? u32x4{w[1], w[2], w[3], w[4]}
                                      : u32x4{align2(w[1], w[0]), align2(w[2], w[1]), align2(w[3], w[2]),
                                              align2(w[4], w[3])};
            *reinterpret_cast<u32x4*>(area + NB_OFF + kpos(cell) * NBR + 16 * blk) = nib;
            const bool valid = cell >= lo_c && cell < hi_c;
            dbits[k] = valid ? (blk_odd ? (w[0] >> 16) : (w[0] & 0xFFFFu)) : 0u;
            vneed = fmaxf(vneed, 8.0f * fabsf(f16v(dbits[k])));
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
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int cell = (lane >> 3) + 8 * k;
            *reinterpret_cast<_Float16*>(area + DV_OFF + (blk * CELLS + kpos(cell)) * 2) =
                (_Float16)(f16v(dbits[k]) * d_mul);
        }

        // ---- context: per block, channels n16 (low nibbles) and n16 + 16 ----
#pragma unroll
        for (int bb = 0; bb < NBLK; ++bb) {
            const i32x2 nb = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (i32x2 __attribute__((address_space(3)))*)(nb_rd + 16 * bb));
            const half8_t dv = *reinterpret_cast<const half8_t*>(dv_rd + 64 * bb);
            const uint32_t x0 = (uint32_t)nb.x, x1 = (uint32_t)nb.y;
            const half8_t vl = nib8(x0 & 0x0F0F0F0Fu, x1 & 0x0F0F0F0Fu);
            const half8_t vh = nib8((x0 >> 4) & 0x0F0F0F0Fu, (x1 >> 4) & 0x0F0F0F0Fu);
            const half8_t bl_h = vl * dv, bh_h = vh * dv;
            const half8_t bl_l = __builtin_elementwise_fma(vl, dv, -bl_h);
            const half8_t bh_l = __builtin_elementwise_fma(vh, dv, -bh_h);
            acc[2 * bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bl_h, acc[2 * bb], 0, 0, 0);
            acc[2 * bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bl_l, acc[2 * bb], 0, 0, 0);
            acc[2 * bb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bh_h, acc[2 * bb + 1], 0, 0, 0);
            acc[2 * bb + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bh_l, acc[2 * bb + 1], 0, 0, 0);
        }
    }

    // ---- a window group on a wave the bulk leaves free ----
    // Window cells u = 32k + c (c < 32) sit in ring slot n_sink + (ovl_ra + u)
    // mod n_ring as exact fp16 rows, so K and V enter the products as they
    // are stored: one MFMA per k-step and per dim tile, and this wave's V
    // scale stays 2^0.  Score tile t row r = cell 16t + r; the score output
    // element (t, i) of lane group g is then cell 16t + 4g + i, the context's
    // k position 8g + 4t + i, and the V operand takes rows 4g + [0, 4) and
    // 16 + 4g + [0, 4) by transpose reads of the staged rows.
    if (a.win_groups > 0) {
        const int64_t k = (int64_t)chunk + (int64_t)wave * n_slices - n_grp;   // (no bulk group: n_grp
        if (k >= 0 && k < a.win_groups) {                                       //  fills one round)
            const int n_wc = (a.n_win - 32 * (int)k < CELLS) ? a.n_win - 32 * (int)k : CELLS;
            auto row_of = [&](int c) -> int {           // byte offset of cell c's row; past n_wc: none
                int rr = a.ovl_ra + 32 * (int)k + c;
                rr = rr % a.n_ring;
                return c < n_wc ? ((a.n_sink + rr) * a.n_kv + kvh) * (D * 2) : a.ovl_bytes;
            };
            const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.k_ovl), (short)0, a.ovl_bytes, kBufWord3);
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(a.v_ovl), (short)0, a.ovl_bytes, kBufWord3);
            u32x4 kop[2][KSTEPS];                       // K operands: channels 32s + 8g .. +8
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int ro = row_of(16 * t + n16);
#pragma unroll
                for (int s = 0; s < KSTEPS; ++s)
                    kop[t][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                              kr, ro + 64 * s + 16 * g, 0, 0));
            }
            u32x4 vrow[CELLS * 2 * D / 16 / 64];        // 16-byte pieces lane + 64 j: cell p / 32, piece p % 32
#pragma unroll
            for (int j = 0; j < CELLS * 2 * D / 16 / 64; ++j) {
                const int p = lane + 64 * j;
                vrow[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                        vr, row_of(p >> 5) + 16 * (p & 31), 0, 0));
            }
            f32x4 sc4[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    sc4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, kop[t][s]),
                                                                    qb[s], sc4[t], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < CELLS * 2 * D / 16 / 64; ++j) {
                const int p = lane + 64 * j;
                *reinterpret_cast<u32x4*>(area + (p >> 5) * WLDR + 16 * (p & 31)) = vrow[j];
            }
            float sc[8];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = sc4[t][i];
                    const float x = (v + xor_lane<1>(v)) * hf;
                    sc[4 * t + i] = (16 * t + 4 * g + i < n_wc) ? x : -INFINITY;
                }
            const half8_t pa = weights(sc);
            const uint8_t* pv = area + (4 * g + (n16 >> 2)) * WLDR + 8 * (n16 & 3);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(pv + 32 * t));
                const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (i16x4 __attribute__((address_space(3)))*)(pv + 16 * WLDR + 32 * t));
                const half8_t B = __builtin_shufflevector(__builtin_bit_cast(half4_t, h0),
                                                          __builtin_bit_cast(half4_t, h1), 0, 1, 2, 3, 4, 5, 6, 7);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, B, acc[t], 0, 0, 0);
            }
        }
    }

    // ---- merge the 8 waves in LDS, add the two rows of each head, write the partial ----
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

// ---------------------------------------------------------------------------
// Combine: one workgroup per (query row, 64-channel slice).  The row's overlay
// cells (sinks [0, n_sink) and the window [ovl_a, T), both cut at the token's
// causal limit) are attended here in f32 from their fp16 copies, in batches
// of 320 overlay cells and 128 bulk partials merged like an online softmax
// (one batch at the pages' sizes).  Per batch: the loads of the overlay K rows
// (8 lanes per cell, lane part k holding channels 32k .. 32k+31 of the query)
// and of the partials are issued first; the scores go to LDS with each cell's
// value-row offset; then the value loads (wave p: the batch's overlay cells
// p, p + 8, ... for its 64 channels) are issued while the batch maximum and
// the weights (one per cell and partial, in LDS) are formed; the weighted
// sums need no branch (cells and partials past the end read 0 with weight 0).
// ---------------------------------------------------------------------------
constexpr int kCombThreads = 512;
constexpr int kCombSlice = 64;
constexpr int NPART = kCombThreads / kCombSlice;    // waves, one context part each
constexpr int kRoundsAll = 5;           // score rounds (64 cells each) per batch: the whole overlay
constexpr int kRoundsSinks = 1;         // the sinks alone (the decode kernel attended the window)
constexpr int kChunksPerWave = 16;
constexpr int JB = NPART * kChunksPerWave;          // bulk partials per batch

struct CombArgs {
    const float* part_acc;      // [n_split][n_qrows][D], bulk partials (m in log2 units)
    const float* part_ml;
    int32_t n_split;
    const float* q;             // [S][Hq][D]
    const uint16_t* k_ovl;      // [n_ovl][n_kv][D] fp16
    const uint16_t* v_ovl;
    int32_t n_ovl;              // overlay slots: n_sink + n_window + n_slack
    float sm_scale;
    int64_t T;
    int64_t pos0;               // < 0: every cell (decode)
    int32_t Hq, n_kv;
    int32_t n_sink;
    int64_t ovl_a;              // first window cell: max(n_sink, T - n_window)
    int32_t ovl_ra, n_ring;     // ring slot of ovl_a, ring length n_window + n_slack
    int32_t win_in_bulk;        // 1: the decode kernel attended the window, only the sinks are left
    float* out;
    float* lse;
};

// ROUNDS = kRoundsSinks: every load of a batch goes out before its first
// wait (the value rows' offsets follow from the cell index, no branch), one
// memory round trip; with kRoundsAll the value loads wait for the scores
// (more than the 63 loads a wave can count in flight otherwise).
template <int ROUNDS>
__global__ __launch_bounds__(kCombThreads) void k_combine_q2k(CombArgs a) {
    constexpr int kRounds = ROUNDS;
    constexpr int CB = kRounds * 64;        // overlay cells per batch
    constexpr int kCellsPerWave = CB / NPART;
    constexpr bool kEarlyV = ROUNDS == kRoundsSinks;
    __shared__ float w_s[CB];               // the batch's overlay scores, then weights
    __shared__ int o_s[CB];                 // their value rows: byte offset of (slot, kvh, c0)
    __shared__ float f_s[JB];               // the batch's partial maxima, then weights
    __shared__ float l_s[JB];               // the batch's partial sums l
    __shared__ float red_s[kCombThreads / 64];
    __shared__ float lp_s[kCombThreads / 64];
    __shared__ float part_s[NPART][kCombSlice];
    const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
    const int64_t r = blockIdx.x;                       // query row: token * Hq + head
    const int tok = (int)(r / a.Hq), h = (int)(r % a.Hq);
    const int kvh = h / (a.Hq / a.n_kv);
    const int64_t n_qrows = gridDim.x;
    const int64_t lim = a.pos0 < 0 ? a.T : a.pos0 + tok + 1;
    const int n_s = (int)(lim < a.n_sink ? lim : a.n_sink);              // sinks attended
    const int n_w = a.win_in_bulk ? 0 : (int)(lim > a.ovl_a ? lim - a.ovl_a : 0);   // window cells attended here
    const int n_ov = n_s + n_w;
    const int n_sp = a.n_split;
    const int c0 = blockIdx.y * kCombSlice;
    const int ovl_bytes = a.n_ovl * a.n_kv * D * 2;
    const __amdgpu_buffer_rsrc_t k_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.k_ovl), (short)0, ovl_bytes, kBufWord3);
    const __amdgpu_buffer_rsrc_t v_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.v_ovl), (short)0, ovl_bytes, kBufWord3);
    // the row's partials of this slice: chunk j, channel c0 + l at byte j pstride + 4 l
    const int pstride = (int)(n_qrows * D * 4);
    const __amdgpu_buffer_rsrc_t p_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.part_acc + r * D + c0), (short)0, n_sp * pstride, kBufWord3);
    const int mstride = (int)(n_qrows * 8);
    const __amdgpu_buffer_rsrc_t m_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.part_ml + r * 2), (short)0, n_sp * mstride, kBufWord3);
    const int j8 = ln >> 3, k8 = ln & 7;                // score lanes: cell j8 of the wave's 8, part k8
    // the query part as loaded (the score factor goes on the finished dot, so
    // the first use of these registers comes after the batch's loads are out:
    // every load of a batch then waits on one memory round trip)
    float qv[32];
    const float qf = a.sm_scale * kLog2e;
    {
        const float* qr = a.q + r * D + 32 * k8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float4 v = *reinterpret_cast<const float4*>(qr + 4 * e);
            qv[4 * e] = v.x; qv[4 * e + 1] = v.y; qv[4 * e + 2] = v.z; qv[4 * e + 3] = v.w;
        }
    }
    const int nb_ov = (n_ov + CB - 1) / CB, nb_sp = (n_sp + JB - 1) / JB;
    const int nb = nb_ov > nb_sp ? nb_ov : nb_sp;
    float acc = 0.0f, lloc = 0.0f, M = -INFINITY;
    for (int bi = 0; bi < nb; ++bi) {
        // overlay K rows of the batch's cells, the partials' (m, l) and values
        int roff[kRounds];
        u32x4 w[kRounds][4];
#pragma unroll
        for (int rd = 0; rd < kRounds; ++rd) {
            const int u = bi * CB + rd * 64 + 8 * wv + j8;
            int rr = a.ovl_ra + (u - n_s);
            rr = rr >= a.n_ring ? rr - a.n_ring : rr;
            const int slot = u < n_s ? u : a.n_sink + rr;
            roff[rd] = u < n_ov ? (slot * a.n_kv + kvh) * (D * 2) : ovl_bytes;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[rd][e] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                       k_rs, roff[rd] + 64 * k8 + 16 * e, 0, 0));
        }
        const int jm = bi * JB + tid;
        const int moff = (tid < JB && jm < n_sp) ? jm * mstride : n_sp * mstride;
        const float mj = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(m_rs, moff, 0, 0));
        const float lj = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(m_rs, moff + 4, 0, 0));
        float vp[kChunksPerWave];
#pragma unroll
        for (int k = 0; k < kChunksPerWave; ++k) {
            const int j = bi * JB + k * NPART + wv;
            vp[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                p_rs, j < n_sp ? j * pstride + 4 * ln : n_sp * pstride, 0, 0));
        }
        float vo[kCellsPerWave];
        if constexpr (kEarlyV) {
            // this wave's overlay cells k NPART + wv (past the row's cells:
            // the end of the buffer, which reads 0)
#pragma unroll
            for (int k = 0; k < kCellsPerWave; ++k) {
                const int u = bi * CB + k * NPART + wv;
                int rr = a.ovl_ra + (u - n_s);
                rr = rr >= a.n_ring ? rr - a.n_ring : rr;
                const int slot = u < n_s ? u : a.n_sink + rr;
                const int off = u < n_ov ? (slot * a.n_kv + kvh) * (D * 2) + 2 * (c0 + ln) : ovl_bytes;
                vo[k] = f16v(__builtin_amdgcn_raw_buffer_load_b16(v_rs, off, 0, 0));
            }
        }
        // scores (-inf past the batch's cells) and value-row offsets
        float mb = -INFINITY;
#pragma unroll
        for (int rd = 0; rd < kRounds; ++rd) {
            float sp = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const u32x4 x = w[rd][e];
                sp = fmaf(qv[8 * e], f16v(x.x & 0xFFFFu), sp);
                sp = fmaf(qv[8 * e + 1], f16v(x.x >> 16), sp);
                sp = fmaf(qv[8 * e + 2], f16v(x.y & 0xFFFFu), sp);
                sp = fmaf(qv[8 * e + 3], f16v(x.y >> 16), sp);
                sp = fmaf(qv[8 * e + 4], f16v(x.z & 0xFFFFu), sp);
                sp = fmaf(qv[8 * e + 5], f16v(x.z >> 16), sp);
                sp = fmaf(qv[8 * e + 6], f16v(x.w & 0xFFFFu), sp);
                sp = fmaf(qv[8 * e + 7], f16v(x.w >> 16), sp);
            }
            sp += xor_lane<1>(sp);
            sp += xor_lane<2>(sp);
            sp += xor_lane<4>(sp);
            sp *= qf;
            const int u = bi * CB + rd * 64 + 8 * wv + j8;
            sp = u < n_ov ? sp : -INFINITY;
            mb = fmaxf(mb, sp);
            if (k8 == 0) {
                w_s[rd * 64 + 8 * wv + j8] = sp;
                o_s[rd * 64 + 8 * wv + j8] = roff[rd] + 2 * c0;
            }
        }
        const float mjv = (tid < JB && jm < n_sp) ? mj : -INFINITY;
        if (tid < JB) {
            f_s[tid] = mjv;
            l_s[tid] = lj;
        }
        mb = wave_max(fmaxf(mb, mjv));
        if (ln == 0) red_s[wv] = mb;
        __syncthreads();                                // scores, offsets, maxima visible
        // value loads of this wave's overlay cells (issued before the weights)
        if constexpr (!kEarlyV) {
#pragma unroll
            for (int k = 0; k < kCellsPerWave; ++k)
                vo[k] = f16v(__builtin_amdgcn_raw_buffer_load_b16(v_rs, o_s[k * NPART + wv] + 2 * ln, 0, 0));
        }
#pragma unroll
        for (int i = 0; i < kCombThreads / 64; ++i) mb = fmaxf(mb, red_s[i]);
        const float Mn = fmaxf(M, mb);
        const float sc = (Mn == -INFINITY || M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        acc *= sc;
        lloc *= sc;
        M = Mn;
        // weights (0 past the end), once per cell and per partial, and the row's sum
        if (tid < CB) {
            const float x = w_s[tid];
            const float wt = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - M);
            w_s[tid] = wt;
            lloc += wt;
        }
        if (tid < JB) {
            const float m = f_s[tid];
            const float ft = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
            f_s[tid] = ft;
            lloc += ft * l_s[tid];
        }
        __syncthreads();                                // weights visible
#pragma unroll
        for (int k = 0; k < kCellsPerWave; ++k) acc = fmaf(w_s[k * NPART + wv], vo[k], acc);
#pragma unroll
        for (int k = 0; k < kChunksPerWave; ++k) acc = fmaf(f_s[k * NPART + wv], vp[k], acc);
        __syncthreads();                                // before the next batch reuses the LDS arrays
    }
    lloc += xor_lane<32>(lloc);
    lloc += xor_lane<16>(lloc);
    lloc += xor_lane<8>(lloc);
    lloc += xor_lane<4>(lloc);
    lloc += xor_lane<2>(lloc);
    lloc += xor_lane<1>(lloc);
    if (ln == 0) lp_s[wv] = lloc;
    part_s[wv][ln] = acc;
    __syncthreads();
    if (wv == 0) {
        float L = 0.0f, sum = 0.0f;
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
            L += lp_s[i];
            sum += part_s[i][ln];
        }
        a.out[r * D + c0 + ln] = L > 0.0f ? sum / L : 0.0f;   // nothing attended: 0 (lse -inf)
        if (a.lse != nullptr && blockIdx.y == 0 && ln == 0)
            a.lse[r] = (M + log2f(L)) * 0.69314718055994531f;
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

namespace {
// overlay geometry of the cache: the first window cell and its ring slot
void overlay_geometry(const kvq_cache& kv, int64_t& ovl_a, int32_t& ovl_ra, int32_t& n_ring) {
    n_ring = kv.n_window + kv.n_slack;
    const int64_t wb = kv.n_rows - kv.n_window;
    ovl_a = wb > kv.n_sink ? wb : kv.n_sink;
    ovl_ra = n_ring > 0 ? (int32_t)((ovl_a - kv.n_sink) % n_ring) : 0;
}
}  // namespace

hipError_t launch_q2k_mfma(const kvq_cache& kv, const AttnPlan& p, const float* q, int32_t Hq,
                           int32_t S, int64_t pos0, float sm_scale, float* part_acc,
                           float* part_ml, float* out, float* lse, hipStream_t s) {
    Q2kArgs a;
    a.k_codes = kv.codes;
    a.k_scale = reinterpret_cast<const uint16_t*>(kv.scales);
    a.v_blocks = kv.v_blocks;
    a.q = q;
    a.sm_scale = sm_scale;
    a.T = kv.n_rows;
    a.S = S;
    a.pos0 = S == 1 && pos0 < 0 ? -1 : pos0;
    a.n_kv = kv.n_kv;
    const bool ovl = (kv.n_sink + kv.n_window) > 0;
    int64_t ovl_a = kv.n_rows;
    int32_t ovl_ra = 0, n_ring = 0;
    if (ovl) overlay_geometry(kv, ovl_a, ovl_ra, n_ring);
    // bulk cells: past the sinks and before the window
    a.bulk_hi = ovl ? (ovl_a < kv.n_rows ? ovl_a : kv.n_rows) : kv.n_rows;
    a.bulk_lo = ovl ? (kv.n_sink < a.bulk_hi ? kv.n_sink : a.bulk_hi) : 0;
    const int blocks = p.n_split * kv.n_kv * S;
    a.xcd_map = (blocks % 8 == 0) ? 1 : 0;
    const Codebook4& cb = codebook4();
    uint32_t lo = 0, hi = 0;
    float amax = 0.0f;
    for (int i = 0; i < 4; ++i) {
        const _Float16 hv = (_Float16)cb.level[i];
        const uint16_t bits = __builtin_bit_cast(uint16_t, hv);
        lo |= (uint32_t)(bits & 0xFFu) << (8 * i);
        hi |= (uint32_t)(bits >> 8) << (8 * i);
        amax = fmaxf(amax, fabsf(cb.level[i]));
    }
    a.lv_lo = lo;
    a.lv_hi = hi;
    a.lv_absmax = amax;
    a.part_acc = part_acc;
    a.part_ml = part_ml;
    // the window on the decode kernel's free waves: one decode token whose
    // bulk groups and window groups fit one round (no wave takes both)
    a.k_ovl = kv.k_ovl;
    a.v_ovl = kv.v_ovl;
    a.ovl_bytes = 0;
    a.n_sink = kv.n_sink;
    a.ovl_ra = ovl_ra;
    a.n_ring = n_ring;
    a.n_win = 0;
    a.win_groups = 0;
    if (ovl && S == 1 && a.pos0 < 0 && kv.n_rows > ovl_a) {
        const int64_t g_first = a.bulk_lo / CELLS;
        const int64_t n_grp = a.bulk_hi > a.bulk_lo ? (a.bulk_hi + CELLS - 1) / CELLS - g_first : 0;
        const int64_t n_win = kv.n_rows - ovl_a;
        const int64_t wg = (n_win + CELLS - 1) / CELLS;
        const int64_t ovl_bytes = ((int64_t)kv.n_sink + n_ring) * kv.n_kv * D * 2;
        if (n_grp + wg <= (int64_t)kWaves * p.n_split && ovl_bytes < (int64_t{1} << 31)) {
            a.ovl_bytes = (int32_t)ovl_bytes;
            a.n_win = (int32_t)n_win;
            a.win_groups = (int32_t)wg;
        }
    }
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = set_dyn_lds_once(reinterpret_cast<const void*>(&k_q2k_mfma), kDynLds, lds_set);
    if (e != hipSuccess) return e;
    k_q2k_mfma<<<blocks, kThreads, kDynLds, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!ovl)
        return launch_combine(KVQ_Q2K, part_acc, part_ml, p.n_split, p.n_qrows, D, 0, true, out, lse, s);
    CombArgs c;
    c.part_acc = part_acc;
    c.part_ml = part_ml;
    c.n_split = p.n_split;
    c.q = q;
    c.k_ovl = kv.k_ovl;
    c.v_ovl = kv.v_ovl;
    c.n_ovl = kv.n_sink + n_ring;
    c.sm_scale = sm_scale;
    c.T = kv.n_rows;
    c.pos0 = a.pos0;
    c.Hq = Hq;
    c.n_kv = kv.n_kv;
    c.n_sink = kv.n_sink;
    c.ovl_a = ovl_a;
    c.ovl_ra = ovl_ra;
    c.n_ring = n_ring;
    c.win_in_bulk = a.win_groups > 0 ? 1 : 0;
    c.out = out;
    c.lse = lse;
    if (c.win_in_bulk && kv.n_sink <= kRoundsSinks * 64)
        k_combine_q2k<kRoundsSinks><<<dim3((unsigned)p.n_qrows, D / kCombSlice), kCombThreads, 0, s>>>(c);
    else
        k_combine_q2k<kRoundsAll><<<dim3((unsigned)p.n_qrows, D / kCombSlice), kCombThreads, 0, s>>>(c);
    return hipGetLastError();
}

}  // namespace kvq
