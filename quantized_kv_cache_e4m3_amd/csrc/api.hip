// extern "C" boundary of libkvq.so: argument checks, workspace sizing,
// dispatch to the kernels, and the library's own codebook construction.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

// Lloyd-Max levels for N(0,1) in double precision: alternate the two
// optimality conditions (boundaries at midpoints, levels at the conditional
// means (phi(a) - phi(b)) / (Phi(b) - Phi(a))) from a uniform start until the
// levels stop moving.  Lloyd (1957), Max (1960).
void lloyd_max(int L, double* c) {
    for (int k = 0; k < L; ++k) c[k] = (k + 0.5 - 0.5 * L) * (4.0 / L);
    const double inv_sqrt2 = 0.70710678118654752440, inv_sqrt2pi = 0.39894228040143267794;
    double b[17];
    for (int it = 0; it < 200000; ++it) {
        b[0] = -INFINITY;
        b[L] = INFINITY;
        for (int k = 1; k < L; ++k) b[k] = 0.5 * (c[k - 1] + c[k]);
        double moved = 0.0;
        for (int k = 0; k < L; ++k) {
            const double lo = b[k], hi = b[k + 1];
            const double plo = isinf(lo) ? 0.0 : exp(-0.5 * lo * lo) * inv_sqrt2pi;
            const double phi = isinf(hi) ? 0.0 : exp(-0.5 * hi * hi) * inv_sqrt2pi;
            const double clo = 0.5 * erfc(-lo * inv_sqrt2), chi = 0.5 * erfc(-hi * inv_sqrt2);
            const double nk = (plo - phi) / (chi - clo);
            moved = fmax(moved, fabs(nk - c[k]));
            c[k] = nk;
        }
        if (moved < 1e-15) break;
    }
}

template <int L>
void build_book(float* level, float* thr) {
    double c[L];
    lloyd_max(L, c);
    for (int k = 0; k < L; ++k) level[k] = (float)(_Float16)c[k];   // RNE to half
    for (int k = 0; k + 1 < L; ++k) thr[k] = (level[k] + level[k + 1]) / 2.0f;
}

Codebook16 g_cb16;
Codebook4 g_cb4;
std::once_flag g_books_once;

void init_books() {
    std::call_once(g_books_once, [] {
        build_book<16>(g_cb16.level, g_cb16.thr);
        build_book<4>(g_cb4.level, g_cb4.thr);
    });
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline bool is_pow2(int64_t n) { return n >= 2 && (n & (n - 1)) == 0; }

kvq_status launch_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_LAUNCH; }

// Shape checks common to both attention entry points.
kvq_status check_cache(const kvq_cache* kv) {
    if (kv == nullptr) return KVQ_ERR_NULL;
    if (kv->n_rows < 1 || kv->d < 1) return KVQ_ERR_SHAPE;
    if (kv->codes == nullptr || kv->scales == nullptr) return KVQ_ERR_NULL;
    switch (kv->fmt) {
        case KVQ_FP8:
            if (kv->n_kv != 1 || kv->d > 1024) return KVQ_ERR_SHAPE;
            if (!aligned(kv->scales, 4)) return KVQ_ERR_ALIGN;
            break;
        case KVQ_TQ4:
            if (kv->n_kv != 1 || !is_pow2(kv->d) || kv->d > 1024) return KVQ_ERR_SHAPE;
            if (!aligned(kv->scales, 4)) return KVQ_ERR_ALIGN;
            break;
        case KVQ_Q2K:
            if (kv->n_kv < 1 || kv->n_kv > 64 || kv->d % 32 != 0 || kv->d > 512 ||
                kv->n_sink < 0 || kv->n_window < 0 || kv->n_sink > 4096 ||
                kv->n_window > 4096 || kv->n_slack < 0 || kv->n_slack > 4096)
                return KVQ_ERR_SHAPE;
            if (kv->v_blocks == nullptr) return KVQ_ERR_NULL;
            if ((kv->n_sink + kv->n_window) > 0 && (kv->k_ovl == nullptr || kv->v_ovl == nullptr))
                return KVQ_ERR_NULL;
            if (!aligned(kv->scales, 2) || !aligned(kv->v_blocks, 2) || !aligned(kv->k_ovl, 2) ||
                !aligned(kv->v_ovl, 2))
                return KVQ_ERR_ALIGN;
            break;
        default:
            return KVQ_ERR_SHAPE;
    }
    if (kv->fmt != KVQ_Q2K && kv->n_slack != 0) return KVQ_ERR_SHAPE;
    // rope part of the MLA key (FP8 / TQ4)
    if (kv->d_rope != 0) {
        if (kv->fmt == KVQ_Q2K || kv->d_rope < 0 || kv->d_rope > 1024) return KVQ_ERR_SHAPE;
        if (kv->fmt == KVQ_TQ4 && (!is_pow2(kv->d_rope) || kv->d_rope < 2)) return KVQ_ERR_SHAPE;
        if (kv->rope_codes == nullptr || kv->rope_scales == nullptr) return KVQ_ERR_NULL;
        if (!aligned(kv->rope_scales, 4)) return KVQ_ERR_ALIGN;
    }
    return KVQ_OK;
}

}  // namespace

kvq_status decode_request(const kvq_cache* kv, const float* q, int32_t n_q_heads, const float* out,
                          const float* lse, AttnPlan& plan) {
    const kvq_status cs = check_cache(kv);
    if (cs != KVQ_OK) return cs;
    if (n_q_heads < 1 || n_q_heads > 4096 || n_q_heads % kv->n_kv != 0) return KVQ_ERR_SHAPE;
    if (q == nullptr || out == nullptr) return KVQ_ERR_NULL;
    if (!aligned(q, 4) || !aligned(out, 4) || !aligned(lse, 4)) return KVQ_ERR_ALIGN;
    plan = make_plan(*kv, n_q_heads, 1, q);
    return KVQ_OK;
}

const Codebook16& codebook16() {
    init_books();
    return g_cb16;
}
const Codebook4& codebook4() {
    init_books();
    return g_cb4;
}

}  // namespace kvq

using namespace kvq;

extern "C" {

const char* kvq_status_str(int32_t status) {
    switch (status) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_NULL: return "a required pointer is NULL";
        case KVQ_ERR_SHAPE: return "a size is out of range or inconsistent";
        case KVQ_ERR_ALIGN: return "a buffer is not aligned as required";
        case KVQ_ERR_WORKSPACE: return "workspace is smaller than attn_workspace_bytes()";
        case KVQ_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
        case KVQ_ERR_UNSUPPORTED: return "request not supported by this library";
        case KVQ_ERR_SCRATCH:
            return "request needs more than the no-allocation scratch (KVQ_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

size_t kvq_row_bytes(int32_t fmt, int32_t d, int32_t n_kv) {
    if (d < 1 || n_kv < 1) return 0;
    switch (fmt) {
        case KVQ_FP8: return (size_t)d + 4;
        case KVQ_TQ4: return (d % 2) ? 0 : (size_t)d / 2 + 4;
        case KVQ_Q2K:
            if (d % 32) return 0;
            return (size_t)n_kv * ((size_t)d / 4 + (size_t)d / 16 + 18 * ((size_t)d / 32));
        default: return 0;
    }
}

kvq_status kvq_codebook(int32_t levels, float* out) {
    if (out == nullptr) return KVQ_ERR_NULL;
    if (levels == 16) {
        for (int i = 0; i < 16; ++i) out[i] = codebook16().level[i];
        return KVQ_OK;
    }
    if (levels == 4) {
        for (int i = 0; i < 4; ++i) out[i] = codebook4().level[i];
        return KVQ_OK;
    }
    return KVQ_ERR_SHAPE;
}

kvq_status kv_encode_fp8(const float* x, int64_t n_rows, int32_t d, uint8_t* codes, float* scales,
                         void* stream) {
    if (n_rows < 0 || d < 1 || d > 65536) return KVQ_ERR_SHAPE;
    if (n_rows == 0) return KVQ_OK;
    if (x == nullptr || codes == nullptr || scales == nullptr) return KVQ_ERR_NULL;
    if (!aligned(x, 4) || !aligned(scales, 4)) return KVQ_ERR_ALIGN;
    return launch_status(launch_encode_fp8(x, n_rows, d, codes, scales, (hipStream_t)stream));
}

kvq_status kv_encode_tq4(const float* x, int64_t n_rows, int32_t d, uint64_t rot_seed,
                         uint8_t* packed, float* radius, void* stream) {
    if (n_rows < 0 || !is_pow2(d) || d > 4096) return KVQ_ERR_SHAPE;
    if (n_rows == 0) return KVQ_OK;
    if (x == nullptr || packed == nullptr || radius == nullptr) return KVQ_ERR_NULL;
    if (!aligned(x, d >= 256 ? 16 : 4) || !aligned(radius, 4)) return KVQ_ERR_ALIGN;
    const int E = d >= 64 ? d / 64 : 1;
    if (!aligned(packed, E >= 8 ? 4 : (E == 4 ? 2 : 1))) return KVQ_ERR_ALIGN;
    return launch_status(launch_encode_tq4(x, n_rows, d, rot_seed, packed, radius, (hipStream_t)stream));
}

kvq_status kv_encode_q2k(const float* k, const float* v, int64_t n_cells, int32_t n_kv, int32_t d,
                         float k_gain, int32_t n_sink, int32_t n_window, uint8_t* k_codes,
                         uint16_t* k_scale, uint8_t* v_blocks, uint16_t* k_ovl, uint16_t* v_ovl,
                         void* stream) {
    if (n_cells < 0 || n_cells % 32 != 0 || n_kv < 1 || n_kv > 64 || d < 32 || d % 32 != 0 ||
        d > 512 || n_sink < 0 || n_window < 0 || n_sink > 4096 || n_window > 4096 ||
        !(k_gain > 0.0f) || isinf(k_gain))
        return KVQ_ERR_SHAPE;
    const bool want_ovl = (n_sink + n_window) > 0;
    if (want_ovl && (k_ovl == nullptr || v_ovl == nullptr)) return KVQ_ERR_NULL;
    if (!want_ovl && (k_ovl != nullptr || v_ovl != nullptr)) return KVQ_ERR_SHAPE;
    if (n_cells == 0 && !want_ovl) return KVQ_OK;
    if (k == nullptr || v == nullptr) return KVQ_ERR_NULL;
    if (n_cells > 0 && (k_codes == nullptr || k_scale == nullptr || v_blocks == nullptr))
        return KVQ_ERR_NULL;
    if (!aligned(k, 4) || !aligned(v, 16) || !aligned(k_codes, 8) || !aligned(k_scale, 2) ||
        !aligned(v_blocks, 2) || !aligned(k_ovl, 2) || !aligned(v_ovl, 2))
        return KVQ_ERR_ALIGN;
    return launch_status(launch_encode_q2k(k, v, n_cells, n_kv, d, k_gain, n_sink, n_window,
                                           k_codes, k_scale, v_blocks, k_ovl, v_ovl,
                                           (hipStream_t)stream));
}

kvq_status kv_append_q2k(const float* k, const float* v, int64_t n_prev, int64_t n_new,
                         int32_t n_kv, int32_t d, float k_gain, int32_t n_sink, int32_t n_window,
                         int32_t n_slack, uint8_t* k_codes, uint16_t* k_scale, uint8_t* v_blocks,
                         uint16_t* k_ovl, uint16_t* v_ovl, void* stream) {
    if (n_prev < 0 || n_new < 0 || n_prev > (int64_t(1) << 40) || n_new > (int64_t(1) << 40) ||
        n_kv < 1 || n_kv > 64 || d < 32 || d % 32 != 0 || d > 512 || n_sink < 0 ||
        n_window < 0 || n_slack < 0 || n_sink > 4096 || n_window > 4096 || n_slack > 4096 ||
        !(k_gain > 0.0f) || isinf(k_gain))
        return KVQ_ERR_SHAPE;
    const bool want_ovl = (n_sink + n_window) > 0;
    if (want_ovl && (k_ovl == nullptr || v_ovl == nullptr)) return KVQ_ERR_NULL;
    if (!want_ovl && (k_ovl != nullptr || v_ovl != nullptr)) return KVQ_ERR_SHAPE;
    if (n_new == 0) return KVQ_OK;
    if (k == nullptr || v == nullptr || k_codes == nullptr || k_scale == nullptr ||
        v_blocks == nullptr)
        return KVQ_ERR_NULL;
    if (!aligned(k, 4) || !aligned(v, 16) || !aligned(k_codes, 8) || !aligned(k_scale, 2) ||
        !aligned(v_blocks, 2) || !aligned(k_ovl, 2) || !aligned(v_ovl, 2))
        return KVQ_ERR_ALIGN;
    return launch_status(launch_append_q2k(k, v, n_prev, n_new, n_kv, d, k_gain, n_sink, n_window,
                                           n_slack, k_codes, k_scale, v_blocks, k_ovl, v_ovl,
                                           (hipStream_t)stream));
}

size_t attn_workspace_bytes(const kvq_cache* kv, int32_t n_q_heads, int32_t n_query_tokens) {
    if (check_cache(kv) != KVQ_OK || n_q_heads < 1 || n_q_heads > 4096 ||
        n_q_heads % kv->n_kv != 0 || n_query_tokens < 1)
        return 0;
    return make_plan(*kv, n_q_heads, n_query_tokens, nullptr).ws_bytes;
}

kvq_status attn_decode_quant(const kvq_cache* kv, const float* q, int32_t n_q_heads, float sm_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
    AttnPlan plan;
    const kvq_status rs = decode_request(kv, q, n_q_heads, out, lse, plan);
    if (rs != KVQ_OK) return rs;
    if (!aligned(ws, 4)) return KVQ_ERR_ALIGN;
    if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return KVQ_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
    return launch_status(launch_attention(*kv, plan, q, 1, n_q_heads, -1, sm_scale, out, lse, ws,
                                          (hipStream_t)stream));
}

kvq_status attn_decode_append_fp8(const kvq_cache* kv, const float* x_new, uint8_t* codes, float* scales,
                                  const float* q, int32_t n_q_heads, float sm_scale, float* out, float* lse,
                                  void* ws, size_t ws_bytes, void* stream) {
    AttnPlan plan;
    const kvq_status rs = decode_request(kv, q, n_q_heads, out, lse, plan);
    if (rs != KVQ_OK) return rs;
    if (kv->fmt != KVQ_FP8) return KVQ_ERR_UNSUPPORTED;
    if (x_new == nullptr || codes == nullptr || scales == nullptr) return KVQ_ERR_NULL;
    if (codes != kv->codes || scales != kv->scales) return KVQ_ERR_SHAPE;
    if (!aligned(x_new, 4) || !aligned(ws, 4)) return KVQ_ERR_ALIGN;
    if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return KVQ_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
    const NewRow nr{x_new, codes, scales, kv->n_rows - 1};
    return launch_status(launch_attention(*kv, plan, q, 1, n_q_heads, -1, sm_scale, out, lse, ws,
                                          (hipStream_t)stream, nullptr, 0, &nr));
}

kvq_status attn_prefill_quant(const kvq_cache* kv, const float* q, int32_t S, int32_t n_q_heads,
                              int64_t pos0, float sm_scale, float* out, float* lse, void* ws,
                              size_t ws_bytes, void* stream) {
    const kvq_status cs = check_cache(kv);
    if (cs != KVQ_OK) return cs;
    if (n_q_heads < 1 || n_q_heads > 4096 || n_q_heads % kv->n_kv != 0) return KVQ_ERR_SHAPE;
    if (S < 1 || pos0 < 0 || pos0 + S > kv->n_rows || (int64_t)S * n_q_heads > (1 << 26))
        return KVQ_ERR_SHAPE;
    if (q == nullptr || out == nullptr) return KVQ_ERR_NULL;
    if (!aligned(q, 4) || !aligned(out, 4) || !aligned(lse, 4) || !aligned(ws, 4)) return KVQ_ERR_ALIGN;
    const AttnPlan plan = make_plan(*kv, n_q_heads, S, q);
    if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return KVQ_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
    return launch_status(launch_attention(*kv, plan, q, S, n_q_heads, pos0, sm_scale, out, lse, ws,
                                          (hipStream_t)stream));
}

// the listed-row view of the cache: the attention sees n_idx rows
static bool gather_view(const kvq_cache* kv, int32_t n_q_heads, int64_t n_idx, const void* q,
                        kvq_cache& g, AttnPlan& p) {
    g = *kv;
    g.n_rows = n_idx;
    if (!mla_mfma_eligible(g, n_q_heads, 1, q)) return false;
    p = AttnPlan{};
    p.path = 1;
    mla_mfma_plan(g, n_q_heads, 1, p, false);   // (listed rows: per head group)
    return true;
}

size_t attn_gather_workspace_bytes(const kvq_cache* kv, int32_t n_q_heads, int64_t n_idx) {
    if (check_cache(kv) != KVQ_OK || n_q_heads < 1 || n_q_heads > 4096 || n_idx < 1 ||
        n_idx > INT32_MAX)
        return 0;
    kvq_cache g;
    AttnPlan p;
    if (!gather_view(kv, n_q_heads, n_idx, reinterpret_cast<const void*>(uintptr_t{16}), g, p))
        return 0;
    return p.ws_bytes;
}

kvq_status attn_decode_gather(const kvq_cache* kv, const int32_t* idx, int64_t n_idx,
                              const float* q, int32_t n_q_heads, float sm_scale, float* out,
                              float* lse, void* ws, size_t ws_bytes, void* stream) {
    const kvq_status cs = check_cache(kv);
    if (cs != KVQ_OK) return cs;
    if (n_q_heads < 1 || n_q_heads > 4096 || n_idx < 1 || n_idx > INT32_MAX) return KVQ_ERR_SHAPE;
    if (idx == nullptr || q == nullptr || out == nullptr) return KVQ_ERR_NULL;
    if (!aligned(idx, 4) || !aligned(q, 4) || !aligned(out, 4) || !aligned(lse, 4))
        return KVQ_ERR_ALIGN;
    kvq_cache g;
    AttnPlan p;
    if (!gather_view(kv, n_q_heads, n_idx, q, g, p)) return KVQ_ERR_UNSUPPORTED;
    if (p.ws_bytes > 0 && (ws == nullptr || ws_bytes < p.ws_bytes)) return KVQ_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return KVQ_ERR_ALIGN;
    return launch_status(launch_attention(g, p, q, 1, n_q_heads, -1, sm_scale, out, lse, ws,
                                          (hipStream_t)stream, idx, kv->n_rows));
}

}  // extern "C"
