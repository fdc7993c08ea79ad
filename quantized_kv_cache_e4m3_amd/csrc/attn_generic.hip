// Attention over an encoded cache: the general path for every format and
// shape (decode and causal chunked prefill), on the f32 vector ALUs.
//
// [colibri #399] "Ready for review" comment / [colibri #553] "What's in it":
// scores are taken against the encoded rows without reconstructing the cache:
//   KV8: u = e4m3(code), the row scale f = s_t stays outside the dot;
//   TQ4: the query is rotated once per head (H D q), u = codebook level,
//        f = r_t / d, and the combined context is unrotated once (D H .);
//   q2k: K = level * channel scale, V = (code-8) * d16 (exact in f32), the
//        fp16 overlay cells read their copies ([Strata #2318] "Summary").
// An MLA key with a rope part ([colibri #553] rebase comment, item 1: the
// kv_lora and qk_rope parts of a row are quantized separately) adds a second
// dot over the rope columns with the rope row's own factor (TQ4: the query's
// rope part rotated with the rope seed); the value stays the latent part.
// One workgroup owns `heads_per_blk` query rows that share one KV head and
// one causal limit, and one chunk of the rows; it runs an online softmax over
// tiles of kTile rows decoded into LDS and writes (m, l, acc) partials.  The
// combine kernel merges the chunks (and unrotates TQ4).
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 16;        // rows decoded into LDS per step
constexpr int kMaxHB = 16;       // query rows per workgroup (at most)
constexpr int64_t kDirectRows = kTile; // a cache of one tile: one chunk, no combine

struct AttnArgs {
    int32_t fmt, d, n_kv, n_sink, n_window;
    int32_t n_slack;             // q2k overlay: window ring = n_window + n_slack slots
    int64_t ovl_a;               // first non-sink window cell, max(n_sink, T - n_window)
    int32_t ovl_ra;              // (ovl_a - n_sink) mod (n_window + n_slack)
    int32_t dr;                  // rope columns of the key (0: none)
    const uint8_t* rcodes;       // rope rows (FP8 [T][dr], TQ4 [T][dr/2])
    const float* rscales;        // rope row scale / radius
    uint64_t rseed;              // TQ4 rope rotation seed
    int64_t T;                   // cached rows (for the overlay position)
    const uint8_t* codes;
    const void* scales;
    const uint8_t* v_blocks;
    const uint16_t* k_ovl;
    const uint16_t* v_ovl;
    uint64_t seed;
    const float* q;
    int32_t S, Hq, hb;           // query tokens, heads, rows per workgroup
    int64_t pos0;
    float sm_scale;
    int32_t n_split;
    int64_t chunk;
    float* part_acc;             // [n_split][n_qrows][d]
    float* part_ml;              // [n_split][n_qrows][2]
    float* out;                  // n_split == 1: [n_qrows][d] written directly
    float* lse;                  // n_split == 1: [n_qrows] or null
};

struct Books {
    float lv16[16];
    float lv4[4];
};

template <int FMT, int DPT>
__global__ __launch_bounds__(kThreads) void k_attn_split(AttnArgs a, Books books) {
    extern __shared__ float smem[];
    const int d = a.d;
    const int dr = a.dr;
    const int dq = d + dr;                         // key (and query) width
    const int ldk = dq + 1;                        // padded row stride (bank spread)
    float* q_s = smem;                             // [hb][dq]
    float* k_s = q_s + a.hb * dq;                  // [kTile][ldk]
    float* v_s = k_s + kTile * ldk;                // [kTile][ldk] (q2k only)
    float* sc_s = v_s + (FMT == KVQ_Q2K ? kTile * ldk : 0);   // [hb][kTile] scores -> weights
    float* f_s = sc_s + kMaxHB * kTile;            // [kTile] row factors
    float* fr_s = f_s + kTile;                     // [kTile] rope row factors
    float* alpha_s = fr_s + kTile;                 // [hb]
    float* m_s = alpha_s + kMaxHB;                 // [hb]
    float* l_s = m_s + kMaxHB;                     // [hb]
    __shared__ float lut_s[16];

    const int tid = threadIdx.x;
    const int hb = a.hb;
    const int qg = blockIdx.x;                     // query-row group
    const int split = blockIdx.y;
    const int r0 = qg * hb;                        // first query row (s * Hq + h)
    const int s_tok = r0 / a.Hq;
    const int h0 = r0 % a.Hq;
    const int group = a.Hq / a.n_kv;
    const int kvh = h0 / group;
    const int64_t lim = (a.S == 1 && a.pos0 < 0) ? a.T : a.pos0 + s_tok + 1;
    const int64_t t_begin = (int64_t)split * a.chunk;
    const int64_t t_end = (t_begin + a.chunk < lim) ? t_begin + a.chunk : lim;

    if (tid < 16) lut_s[tid] = (FMT == KVQ_TQ4) ? books.lv16[tid] : (tid < 4 ? books.lv4[tid] : 0.0f);
    // query rows -> LDS
    for (int i = tid; i < hb * dq; i += kThreads) q_s[i] = a.q[(int64_t)r0 * dq + i];
    if (tid < hb) {
        m_s[tid] = -INFINITY;
        l_s[tid] = 0.0f;
    }
    __syncthreads();
    if constexpr (FMT == KVQ_TQ4) {
        // q' = H D q (unnormalised), once per head; the rope columns [d, dq)
        // are rotated on their own with the rope seed
        for (int i = tid; i < hb * dq; i += kThreads) {
            const int c = i % dq;
            const bool rope = c >= d;
            const int cc = rope ? c - d : c;
            const uint64_t w = splitmix64_at(rope ? a.rseed : a.seed, (uint64_t)(cc >> 6));
            if ((w >> (cc & 63)) & 1ull) q_s[i] = -q_s[i];
        }
        __syncthreads();
        for (int part = 0; part < (dr > 0 ? 2 : 1); ++part) {
            const int n = part ? dr : d, off = part ? d : 0;
            for (int h = 1; h < n; h <<= 1) {
                for (int pidx = tid; pidx < hb * (n / 2); pidx += kThreads) {
                    const int row = pidx / (n / 2), pr = pidx % (n / 2);
                    const int i = (pr / h) * 2 * h + (pr % h);
                    float* qr = q_s + row * dq + off;
                    const float x0 = qr[i], x1 = qr[i + h];
                    qr[i] = x0 + x1;
                    qr[i + h] = x0 - x1;
                }
                __syncthreads();
            }
        }
    }

    float acc[kMaxHB][DPT];
#pragma unroll
    for (int h = 0; h < kMaxHB; ++h)
#pragma unroll
        for (int j = 0; j < DPT; ++j) acc[h][j] = 0.0f;

    for (int64_t t0 = t_begin; t0 < t_end; t0 += kTile) {
        const int nt = (int)((t_end - t0) < kTile ? (t_end - t0) : kTile);
        // ---- decode the tile into LDS (values u and row factors f) ----
        for (int i = tid; i < nt * d; i += kThreads) {
            const int tt = i / d, c = i % d;
            const int64_t t = t0 + tt;
            float ku, vu = 0.0f;
            if constexpr (FMT == KVQ_FP8) {
                ku = e4m3_to_f32(a.codes[t * d + c]);
            } else if constexpr (FMT == KVQ_TQ4) {
                const uint8_t b = a.codes[t * (d / 2) + (c >> 1)];
                ku = lut_s[(c & 1) ? (b >> 4) : (b & 15)];
            } else {
                const int64_t T = a.T;
                int64_t slot = -1;
                if (t < a.n_sink) {
                    slot = t;
                } else if (t >= a.ovl_a) {              // ring slot n_sink + (t - n_sink) mod R
                    const int R = a.n_window + a.n_slack;
                    int r = a.ovl_ra + (int)(t - a.ovl_a);
                    slot = a.n_sink + (r >= R ? r - R : r);
                }
                if (slot >= 0) {
                    const int64_t o = (slot * a.n_kv + kvh) * d + c;
                    ku = f16_bits_to_f32(a.k_ovl[o]);
                    vu = f16_bits_to_f32(a.v_ovl[o]);
                } else {
                    const int64_t g = t >> 5;
                    const int j = (int)(t & 31);
                    const int64_t kc = (g * a.n_kv + kvh) * d + c;
                    const uint32_t byte = a.codes[kc * 8 + (j >> 2)];
                    const uint32_t code = (byte >> (2 * (j & 3))) & 3u;
                    const float ks = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.scales)[kc]);
                    ku = lut_s[code] * ks;
                    const uint8_t* blk = a.v_blocks + ((t * a.n_kv + kvh) * (d / 32) + (c >> 5)) * 18;
                    const float dv = f16_bits_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
                    const int e = c & 31;
                    const uint32_t nib = e < 16 ? (blk[2 + e] & 15u) : (blk[2 + e - 16] >> 4);
                    vu = (float)((int)nib - 8) * dv;
                }
            }
            k_s[tt * ldk + c] = ku;
            if constexpr (FMT == KVQ_Q2K) v_s[tt * ldk + c] = vu;
        }
        if constexpr (FMT != KVQ_Q2K) {
            // rope columns of the key
            for (int i = tid; i < nt * dr; i += kThreads) {
                const int tt = i / dr, c = i % dr;
                const int64_t t = t0 + tt;
                float ku;
                if constexpr (FMT == KVQ_FP8) {
                    ku = e4m3_to_f32(a.rcodes[t * dr + c]);
                } else {
                    const uint8_t b = a.rcodes[t * (dr / 2) + (c >> 1)];
                    ku = lut_s[(c & 1) ? (b >> 4) : (b & 15)];
                }
                k_s[tt * ldk + d + c] = ku;
            }
        }
        if (tid < nt) {
            const int64_t t = t0 + tid;
            float f = 1.0f, fr = 0.0f;
            if constexpr (FMT == KVQ_FP8) f = reinterpret_cast<const float*>(a.scales)[t];
            if constexpr (FMT == KVQ_TQ4) f = reinterpret_cast<const float*>(a.scales)[t] / (float)d;
            if (dr > 0) {
                if constexpr (FMT == KVQ_FP8) fr = a.rscales[t];
                if constexpr (FMT == KVQ_TQ4) fr = a.rscales[t] / (float)dr;
            }
            f_s[tid] = f;
            fr_s[tid] = fr;
        }
        __syncthreads();
        // ---- scores: one (head, row) pair per thread ----
        {
            const int h = tid / kTile, tt = tid % kTile;
            if (h < hb) {
                float sc = -INFINITY;
                if (tt < nt) {
                    const float* qr = q_s + h * dq;
                    const float* kr = k_s + tt * ldk;
                    // four independent partial sums (the LDS reads of one do not
                    // wait for the previous product), added at the end
                    float d4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                    int c = 0;
                    for (; c + 4 <= d; c += 4) {
#pragma unroll
                        for (int k = 0; k < 4; ++k) d4[k] = fmaf(qr[c + k], kr[c + k], d4[k]);
                    }
                    for (; c < d; ++c) d4[0] = fmaf(qr[c], kr[c], d4[0]);
                    const float dot = (d4[0] + d4[1]) + (d4[2] + d4[3]);
                    if (dr > 0) {
                        float dot_r = 0.0f;
                        for (int c = d; c < dq; ++c) dot_r = fmaf(qr[c], kr[c], dot_r);
                        sc = a.sm_scale * (f_s[tt] * dot + fr_s[tt] * dot_r);
                    } else {
                        sc = a.sm_scale * (f_s[tt] * dot);
                    }
                }
                sc_s[h * kTile + tt] = sc;
            }
        }
        __syncthreads();
        // ---- online softmax update per head ----
        if (tid < hb) {
            const int h = tid;
            float mx = m_s[h];
            for (int tt = 0; tt < nt; ++tt) mx = fmaxf(mx, sc_s[h * kTile + tt]);
            const float alpha = (m_s[h] == -INFINITY) ? 0.0f : expf(m_s[h] - mx);
            float lsum = 0.0f;
            for (int tt = 0; tt < kTile; ++tt) {
                const float p = tt < nt ? expf(sc_s[h * kTile + tt] - mx) : 0.0f;
                lsum += p;
                sc_s[h * kTile + tt] = (FMT == KVQ_Q2K) ? p : p * f_s[tt < nt ? tt : 0];
            }
            l_s[h] = l_s[h] * alpha + lsum;
            m_s[h] = mx;
            alpha_s[h] = alpha;
        }
        __syncthreads();
        // ---- context: acc[h][c] = alpha * acc + sum_t w[h][t] * u[t][c] ----
        {
            const float* vsrc = (FMT == KVQ_Q2K) ? v_s : k_s;
#pragma unroll
            for (int h = 0; h < kMaxHB; ++h) {
                if (h < hb) {
                    const float al = alpha_s[h];
#pragma unroll
                    for (int j = 0; j < DPT; ++j) acc[h][j] *= al;
                }
            }
            for (int tt = 0; tt < nt; ++tt) {
#pragma unroll
                for (int j = 0; j < DPT; ++j) {
                    const int c = tid + j * kThreads;
                    const float u = c < d ? vsrc[tt * ldk + c] : 0.0f;
#pragma unroll
                    for (int h = 0; h < kMaxHB; ++h)
                        if (h < hb) acc[h][j] = fmaf(sc_s[h * kTile + tt], u, acc[h][j]);
                }
            }
        }
        __syncthreads();
    }

    const int64_t n_qrows = (int64_t)a.S * a.Hq;
    if (a.n_split == 1) {
        // one chunk: the normalised context and lse (no row at all: 0, -inf)
        for (int h = 0; h < hb; ++h) {
            const float l = l_s[h];
#pragma unroll
            for (int j = 0; j < DPT; ++j) {
                const int c = tid + j * kThreads;
                if (c < d) a.out[((int64_t)r0 + h) * d + c] = l > 0.0f ? acc[h][j] / l : 0.0f;
            }
        }
        if (a.lse != nullptr && tid < hb) a.lse[r0 + tid] = m_s[tid] + logf(l_s[tid]);
        return;
    }
    // ---- partials ----
    for (int h = 0; h < hb; ++h) {
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int c = tid + j * kThreads;
            if (c < d) a.part_acc[((int64_t)split * n_qrows + r0 + h) * d + c] = acc[h][j];
        }
    }
    if (tid < hb) {
        float* ml = a.part_ml + ((int64_t)split * n_qrows + r0 + tid) * 2;
        ml[0] = m_s[tid];
        ml[1] = l_s[tid];
    }
}

// dynamic LDS of k_attn_split: query rows, key (and q2k value) tile, scores,
// row factors, softmax state
size_t split_lds_bytes(int fmt, int d, int dr, int hb) {
    const size_t dq = (size_t)d + dr;
    return sizeof(float) * ((size_t)hb * dq + (size_t)kTile * (dq + 1) * (fmt == KVQ_Q2K ? 2 : 1) +
                            (size_t)kMaxHB * kTile + 2 * kTile + 3 * kMaxHB);
}
constexpr size_t kLdsMax = 160 * 1024;

template <int FMT, int DPT>
hipError_t launch_split_t(const AttnArgs& a, int n_qgroups, hipStream_t s) {
    const size_t lds = split_lds_bytes(FMT, a.d, a.dr, a.hb);
    if (lds > kLdsMax) return hipErrorInvalidValue;
    const dim3 grid(n_qgroups, a.n_split);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_attn_split<FMT, DPT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    Books books;
    const Codebook16& c16 = codebook16();
    const Codebook4& c4 = codebook4();
    for (int i = 0; i < 16; ++i) books.lv16[i] = c16.level[i];
    for (int i = 0; i < 4; ++i) books.lv4[i] = c4.level[i];
    k_attn_split<FMT, DPT><<<grid, kThreads, lds, s>>>(a, books);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const AttnArgs& a, int n_qgroups, hipStream_t s) {
    if (a.d <= 256) return launch_split_t<FMT, 1>(a, n_qgroups, s);
    if (a.d <= 512) return launch_split_t<FMT, 2>(a, n_qgroups, s);
    return launch_split_t<FMT, 4>(a, n_qgroups, s);
}

}  // namespace

AttnPlan make_plan(const kvq_cache& kv, int32_t Hq, int32_t S, const void* q, bool wide_decode) {
    const AttnPlan g = generic_plan(kv, Hq, S);
    // sizing without a query: assume the fast path, reserve enough for either
    const void* qa = q != nullptr ? q : reinterpret_cast<const void*>(uintptr_t{16});
    if (q2k_mfma_eligible(kv, Hq, S, qa)) {
        AttnPlan p{};
        q2k_mfma_plan(kv, Hq, S, p);
        if (q == nullptr && g.ws_bytes > p.ws_bytes) p.ws_bytes = g.ws_bytes;
        return p;
    }
    if (!mla_mfma_eligible(kv, Hq, S, qa)) return g;
    AttnPlan p{};
    p.path = 1;
    mla_mfma_plan(kv, Hq, S, p, wide_decode);
    if (q == nullptr && g.ws_bytes > p.ws_bytes) p.ws_bytes = g.ws_bytes;
    return p;
}

AttnPlan generic_plan(const kvq_cache& kv, int32_t Hq, int32_t S) {
    AttnPlan p{};
    p.n_qrows = Hq * S;
    const int group = Hq / kv.n_kv;
    int hb = kMaxHB;
    while (hb > 1 && (group % hb) != 0) hb >>= 1;
    // wide keys (a rope part on a wide latent): fewer query rows per workgroup
    const int dr = kv.fmt == KVQ_Q2K ? 0 : kv.d_rope;
    while (hb > 1 && split_lds_bytes(kv.fmt, kv.d, dr, hb) > kLdsMax) hb >>= 1;
    p.heads_per_blk = hb;
    p.n_qgroups = p.n_qrows / hb;
    // enough workgroups to cover the 256 CUs twice; chunks in whole tiles
    // (q2k: whole 32-cell groups are not needed by this path)
    const int64_t T = kv.n_rows;
    int64_t want = (512 + p.n_qgroups - 1) / p.n_qgroups;
    const int64_t max_split = (T + kTile - 1) / kTile;
    // a cache of one tile is one chunk: the workgroup writes the output
    // itself, which saves the combine launch (longer caches are faster split:
    // a workgroup walks its tiles one after another)
    if (T <= kDirectRows) want = 1;
    if (want > max_split) want = max_split;
    if (want > 1024) want = 1024;
    if (want < 1) want = 1;
    int64_t chunk = (T + want - 1) / want;
    chunk = ((chunk + kTile - 1) / kTile) * kTile;
    p.chunk = chunk;
    p.n_split = (int32_t)((T + chunk - 1) / chunk);
    p.ws_bytes = (size_t)p.n_split * p.n_qrows * ((size_t)kv.d + 2) * sizeof(float);
    return p;
}

hipError_t launch_attention(const kvq_cache& kv, const AttnPlan& plan, const float* q, int32_t S,
                            int32_t Hq, int64_t pos0, float sm_scale, float* out, float* lse,
                            void* ws, hipStream_t s, const int32_t* idx, int64_t n_cache,
                            const NewRow* nr) {
    if (idx != nullptr && plan.path != 1) return hipErrorInvalidValue;
    if (nr != nullptr) {
        if (kv.fmt != KVQ_FP8 || nr->row < 0 || nr->row >= kv.n_rows) return hipErrorInvalidValue;
        if (!mla_append_fusable(kv, plan, Hq, S, pos0, idx, nr)) {
            const hipError_t e = launch_encode_fp8(nr->x, 1, kv.d, nr->codes + nr->row * kv.d,
                                                   nr->scales + nr->row, s);
            if (e != hipSuccess) return e;
            nr = nullptr;
        }
    }
    if (plan.path == 1) {
        float* part_acc = reinterpret_cast<float*>(ws);
        float* part_ml = part_acc + (size_t)plan.n_split * plan.n_qrows * kv.d;
        hipError_t e = launch_mla_mfma(kv, plan, q, Hq, S, pos0, sm_scale, part_acc, part_ml,
                                       out, lse, s, idx, n_cache, nr);
        if (e != hipSuccess) return e;
        if (plan.n_split == 1)
            return kv.fmt == KVQ_TQ4 ? launch_unrotate(out, plan.n_qrows, kv.d, kv.rot_seed, s)
                                     : hipSuccess;
        return launch_combine(kv.fmt, part_acc, part_ml, plan.n_split, plan.n_qrows, kv.d,
                              kv.rot_seed, plan.log2_domain != 0, out, lse, s);
    }
    if (plan.path == 2) {
        float* part_acc = reinterpret_cast<float*>(ws);
        float* part_ml = part_acc + (size_t)plan.n_split * plan.n_qrows * kv.d;
        return launch_q2k_mfma(kv, plan, q, Hq, S, pos0, sm_scale, part_acc, part_ml, out, lse, s);
    }
    AttnArgs a{};
    a.fmt = kv.fmt;
    a.d = kv.d;
    a.n_kv = kv.n_kv;
    a.n_sink = kv.n_sink;
    a.n_window = kv.n_window;
    a.dr = kv.fmt == KVQ_Q2K ? 0 : kv.d_rope;
    a.n_slack = kv.n_slack;
    {
        const int64_t wb = kv.n_rows - kv.n_window;
        const int64_t R = (int64_t)kv.n_window + kv.n_slack;
        a.ovl_a = wb > kv.n_sink ? wb : kv.n_sink;
        a.ovl_ra = R > 0 ? (int32_t)((a.ovl_a - kv.n_sink) % R) : 0;
    }
    a.rcodes = kv.rope_codes;
    a.rscales = kv.rope_scales;
    a.rseed = kv.rope_seed;
    a.T = kv.n_rows;
    a.codes = kv.codes;
    a.scales = kv.scales;
    a.v_blocks = kv.v_blocks;
    a.k_ovl = kv.k_ovl;
    a.v_ovl = kv.v_ovl;
    a.seed = kv.rot_seed;
    a.q = q;
    a.S = S;
    a.Hq = Hq;
    a.hb = plan.heads_per_blk;
    a.pos0 = pos0;
    a.sm_scale = sm_scale;
    a.n_split = plan.n_split;
    a.chunk = plan.chunk;
    a.part_acc = reinterpret_cast<float*>(ws);
    a.part_ml = a.part_acc + (size_t)plan.n_split * plan.n_qrows * kv.d;
    a.out = out;
    a.lse = lse;
    if (kv.fmt == KVQ_Q2K && (kv.n_sink + kv.n_window) == 0) {
        a.k_ovl = nullptr;
        a.v_ovl = nullptr;
    }
    hipError_t e;
    switch (kv.fmt) {
        case KVQ_FP8: e = launch_fmt<KVQ_FP8>(a, plan.n_qgroups, s); break;
        case KVQ_TQ4: e = launch_fmt<KVQ_TQ4>(a, plan.n_qgroups, s); break;
        default: e = launch_fmt<KVQ_Q2K>(a, plan.n_qgroups, s); break;
    }
    if (e != hipSuccess) return e;
    if (plan.n_split == 1)
        return kv.fmt == KVQ_TQ4 ? launch_unrotate(out, plan.n_qrows, kv.d, kv.rot_seed, s)
                                 : hipSuccess;
    return launch_combine(kv.fmt, a.part_acc, a.part_ml, plan.n_split, plan.n_qrows, kv.d,
                          kv.rot_seed, false, out, lse, s);
}

}  // namespace kvq
