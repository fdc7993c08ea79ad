/*
 * kvq.h - C ABI of libkvq.so: quantized KV-cache encoders and attention that
 * reads the encoded rows directly (gfx950 / MI355X).
 *
 * Pages cited (titles abbreviated):
 *   [colibri #399]  "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant (KV_TQ)
 *                    on CPU, CUDA, and Metal"
 *   [colibri #553]  "CPU: KV cache quantization - KV8 (fp8 e4m3) + KV_TQ
 *                    (rotated-int4 / PolarQuant)"
 *   [Strata #2318]  "KV cache: FP16 sliding window + attention sinks, and an
 *                    optional 2-bit K / 4-bit V cache scheme (--kv q2k)"
 *
 * Conventions for every entry point
 *   - Every buffer argument is a DEVICE pointer owned by the caller; the library
 *     allocates nothing, frees nothing and keeps no per-call state (the one
 *     exception, attn_decode_quant_noalloc, uses a device array that is part
 *     of the library itself; see its declaration).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued on it; no call synchronises.
 *   - Arguments are checked on the host before anything is enqueued.  On any
 *     error nothing is written and the status says why (kvq_status_str()).
 *     A failed kernel launch returns KVQ_ERR_LAUNCH.  No C++ exception crosses
 *     this boundary and there is no fallback path.
 *   - Buffers are laid out densely as described per argument (row-major, last
 *     index fastest) and aligned to their element size; a few inputs need
 *     more, stated per call (KVQ_ERR_ALIGN otherwise).
 *   - Preconditions that are NOT checked on the device: inputs are finite;
 *     q2k inputs (and B times their group RMS) fit in fp16; caches handed to
 *     the attention calls were written by this library's encoders.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_NULL = 1,         /* a required pointer is NULL */
    KVQ_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
    KVQ_ERR_ALIGN = 3,        /* a buffer is not aligned as its call requires */
    KVQ_ERR_WORKSPACE = 4,    /* workspace smaller than attn_workspace_bytes() */
    KVQ_ERR_LAUNCH = 5,       /* the HIP runtime refused a launch */
    KVQ_ERR_UNSUPPORTED = 6,  /* valid request the library does not implement */
    KVQ_ERR_SCRATCH = 7       /* attn_decode_quant_noalloc: the request needs more
                                 than KVQ_NOALLOC_SCRATCH_BYTES of scratch */
} kvq_status;

typedef enum kvq_format {
    KVQ_FP8 = 1,   /* KV8: fp8 e4m3 codes + f32 scale per row      [colibri #399] */
    KVQ_TQ4 = 2,   /* rotated-int4: nibbles + f32 radius per row   [colibri #399] */
    KVQ_Q2K = 3    /* 2-bit K per channel + q4_0 V + fp16 overlay  [Strata #2318] */
} kvq_format;

/* ------------------------------------------------------------------------
 * Encoders (the producer side)
 * ------------------------------------------------------------------------ */

/* KV8 row encoder.  [colibri #399] "Summary" and "Commits" item 1: fp8 e4m3,
 * round to nearest even, one f32 scale per row equal to amax/448;
 * [colibri #553] "What's in it".
 *   x       f32 [n_rows][d]   rows to encode
 *   codes   u8  [n_rows][d]   out: e4m3 byte of x[i] / scale (sign kept,
 *                             magnitudes above 448 saturate to 448)
 *   scales  f32 [n_rows]      out: fl32(max_i |x[i]| / 448); a zero row stores
 *                             scale 0 and all-zero codes
 * To append rows to a cache, pass codes/scales offset to the first new row.
 * Limits: n_rows >= 0, 1 <= d <= 65536. */
kvq_status kv_encode_fp8(const float* x, int64_t n_rows, int32_t d,
                         uint8_t* codes, float* scales, void* stream);

/* Rotated-int4 (TQ4) row encoder.  [colibri #399] "Why rotated-int4 for the
 * 4-bit tier": randomized Hadamard rotation (+-1 diagonal, then Walsh-Hadamard),
 * fixed 16-level N(0,1) Lloyd-Max codebook scaled by radius/sqrt(n), packed
 * nibbles; [colibri #553] rebase comment: widths that are not a power of two
 * are refused (KVQ_ERR_SHAPE), never encoded as garbage.
 *   x         f32 [n_rows][d]    rows; d a power of two, 2 <= d <= 4096;
 *                                16-byte aligned when d >= 256 (packed: 4-byte
 *                                aligned when d >= 512, 2-byte when d = 256)
 *   rot_seed  seed of the sign diagonal: sign i is -1 iff bit (i mod 64) of
 *             SplitMix64 output floor(i/64) (from state rot_seed) is set
 *   packed    u8  [n_rows][d/2]  out: level of element 2j in the low nibble
 *                                of byte j, element 2j+1 in the high nibble
 *   radius    f32 [n_rows]       out: ||x||_2 (fixed pairwise tree); a zero
 *                                radius stores all-zero bytes (inert row)
 * The level of y_i (y = H D x, unnormalised) is the count of thresholds
 * fl32(tau_k * radius) below it, tau_k the midpoints of the f16-rounded
 * codebook. */
kvq_status kv_encode_tq4(const float* x, int64_t n_rows, int32_t d, uint64_t rot_seed,
                         uint8_t* packed, float* radius, void* stream);

/* q2k cache encoder for cells [0, n_cells).  [Strata #2318] "Summary" items
 * 1-3, "Why per-channel K and per-token V", "Memory":
 *   k, v      f32 [n_cells][n_kv][d]; n_cells a multiple of 32 (whole groups),
 *             d a multiple of 32, 32 <= d <= 512, 1 <= n_kv <= 64; v 16-byte
 *             aligned, k_codes 8-byte aligned
 *   k_gain    B: the stored K scale is f16(B * rule); codes use the un-gained
 *             rule (B = 1.10 on the page)
 *   n_sink, n_window  fp16 overlay: cells t < n_sink and t >= n_cells -
 *             n_window keep exact fp16 copies (0 <= each <= 4096)
 *   k_codes   u8  [n_cells/32][n_kv][d][8]  out: 2-bit codes of a channel's
 *             32 cells, cell j of the group in bits 2*(j%4) of byte j/4
 *   k_scale   u16 [n_cells/32][n_kv][d]     out: fp16 scale B * RMS of the
 *             channel over the group (RMS from a cell-order f32 sum of squares)
 *   v_blocks  u8  [n_cells][n_kv][d/32][18] out: q4_0 blocks: fp16 d =
 *             f16(amax/7) little-endian, then 16 bytes, element j<16 in the
 *             low nibble of byte j, element j>=16 in the high nibble of byte
 *             j-16; value (code-8)*d
 *   k_ovl, v_ovl  u16 [n_sink+n_window][n_kv][d] out: fp16 copies; slot s <
 *             n_sink holds cell s, a later cell t the ring slot n_sink +
 *             (t - n_sink) mod n_window (kv_append_q2k with n_slack = 0);
 *             slots no cell reaches are zero.  Both NULL (allowed only when
 *             n_sink = n_window = 0) skip the overlay. */
kvq_status kv_encode_q2k(const float* k, const float* v, int64_t n_cells, int32_t n_kv,
                         int32_t d, float k_gain, int32_t n_sink, int32_t n_window,
                         uint8_t* k_codes, uint16_t* k_scale, uint8_t* v_blocks,
                         uint16_t* k_ovl, uint16_t* v_ovl, void* stream);

/* Append cells [n_prev, n_prev + n_new) to a q2k cache -- decode steps,
 * speculative-verify windows, prefill chunks that start or end mid-group.
 * [Strata #2318] "Attention error under the engine's append patterns" and
 * "Review fixes": every 32-cell group the call touches is requantized from
 * all of its cells present so far; a whole group takes the RMS rule of
 * kv_encode_q2k, a partial group is shrunk toward the previous group's
 * scale, s = sqrt((ss + (32 - n) prev^2) / 32) over its n cells (prev = the
 * previous group's stored scale / k_gain), and the first group, partial, takes
 * the RMS of its cells.  Codes of cells not yet present are 0.  Any split of
 * the same cells into calls stores the same bytes; whole groups appended from
 * an empty cache store what kv_encode_q2k stores (with n_slack = 0).
 * The fp16 overlay is a ring: a sink keeps slot t, any other cell t lives in
 * slot n_sink + (t - n_sink) mod (n_window + n_slack); the slack (16 on the
 * page) lets cells be written ahead of the window's end without evicting a
 * cell still in the window.  Only the sinks and the last n_window + n_slack
 * cells of each call are written, so one call or many leave the same slots.
 *   k, v      f32 [n_prev + n_new][n_kv][d] device: every cell so far (K is
 *             read from the first touched group's first cell, V of the new
 *             cells only)
 *   k_codes, k_scale  as kv_encode_q2k, for ceil((n_prev + n_new)/32)
 *             groups; groups before the touched ones are not written, the
 *             scale of the group before them is read
 *   v_blocks  as kv_encode_q2k, for whole groups: 32 * ceil((n_prev +
 *             n_new)/32) cells (attention reads the last group whole and
 *             masks its absent cells)
 *   k_ovl, v_ovl  u16 [n_sink + n_window + n_slack][n_kv][d], NULL iff
 *             n_sink = n_window = 0
 * Sizes and alignment as kv_encode_q2k; 0 <= n_slack <= 4096, n_new >= 0
 * (0: nothing to do).  Attention reads the result as a kvq_cache with n_rows
 * = n_prev + n_new and this n_slack. */
kvq_status kv_append_q2k(const float* k, const float* v, int64_t n_prev, int64_t n_new,
                         int32_t n_kv, int32_t d, float k_gain, int32_t n_sink,
                         int32_t n_window, int32_t n_slack, uint8_t* k_codes,
                         uint16_t* k_scale, uint8_t* v_blocks, uint16_t* k_ovl,
                         uint16_t* v_ovl, void* stream);

/* ------------------------------------------------------------------------
 * Attention over an encoded cache (the consumer side)
 * ------------------------------------------------------------------------ */

/* A read-only view of one encoded cache.  Pointers as written by the encoders.
 *
 * MLA rope part (FP8 / TQ4 only).  [colibri #553] rebase comment, item 1: a
 * cached MLA row has a kv_lora part and a qk_rope part (512 and 64 wide on
 * that page's model), each quantized on its own -- for TQ4 each rotated on
 * its own, so both widths are powers of two.  With d_rope > 0 the key of row
 * t is its latent part followed by its rope part, the value is the latent
 * part alone, and the query rows are d + d_rope wide (latent part first):
 *   score_t = sm_scale * (q_lat . k_lat_t + q_rope . k_rope_t).
 * The rope rows are encoded by the same format's encoder at width d_rope
 * (kv_encode_fp8, or kv_encode_tq4 with its own seed rope_seed). */
typedef struct kvq_cache {
    int32_t fmt;            /* kvq_format */
    int32_t d;              /* row width: latent width (FP8/TQ4), head dim (Q2K) */
    int32_t n_kv;           /* KV heads: must be 1 for FP8/TQ4 (MLA latent) */
    int32_t n_sink;         /* Q2K overlay sinks (0 for FP8/TQ4) */
    int32_t n_window;       /* Q2K overlay window (0 for FP8/TQ4) */
    int32_t d_rope;         /* FP8/TQ4: width of the key's rope part, 0 = none
                               (<= 1024; TQ4: a power of two >= 2); Q2K: 0 */
    int64_t n_rows;         /* cached rows (cells present; Q2K: any count, the
                               last group may be partial after appends, its
                               buffers sized for the whole group) */
    const uint8_t* codes;   /* FP8: [n_rows][d]; TQ4: [n_rows][d/2]; Q2K: k_codes */
    const void* scales;     /* FP8: f32 scale; TQ4: f32 radius [n_rows]; Q2K: u16 k_scale */
    const uint8_t* v_blocks;   /* Q2K only */
    const uint16_t* k_ovl;     /* Q2K only; NULL iff n_sink = n_window = 0 */
    const uint16_t* v_ovl;     /* Q2K only */
    uint64_t rot_seed;         /* TQ4 only: the seed the rows were encoded with */
    const uint8_t* rope_codes; /* d_rope > 0: FP8 [n_rows][d_rope]; TQ4 [n_rows][d_rope/2] */
    const float* rope_scales;  /* d_rope > 0: FP8 scale / TQ4 radius [n_rows] */
    uint64_t rope_seed;        /* TQ4 with d_rope > 0: the rope rows' seed */
    int32_t n_slack;           /* Q2K: overlay ring slack (0 for kv_encode_q2k
                                  caches; as passed to kv_append_q2k); else 0 */
    int32_t reserved;
} kvq_cache;

/* Bytes of device workspace attn_decode_quant / attn_prefill_quant need for
 * this cache and query shape (0 is possible).  n_query_tokens = 1 for decode. */
size_t attn_workspace_bytes(const kvq_cache* kv, int32_t n_q_heads, int32_t n_query_tokens);

/* One-token attention over every cached row.  [colibri #399] "Ready for
 * review" comment and [colibri #553] "What's in it": scores are taken against
 * the encoded rows (KV8: e4m3 values, the row scale outside the dot; TQ4: the
 * query rotated once per head, dotted with codebook values, the context
 * unrotated once); online softmax over T split into chunks, then a combine
 * step; the MLA latent row is both key and value.  [Strata #2318]: q2k reads K
 * as level * channel scale and V as (code-8)*d, overlay cells as their fp16
 * copies; query head h reads KV head h / (n_q_heads / n_kv).
 *   q     f32 [n_q_heads][d + d_rope]  (see kvq_cache for the rope part)
 *   out   f32 [n_q_heads][d]   out: softmax(sm_scale * q.K^T) V
 *   lse   f32 [n_q_heads]      out (may be NULL): max score + ln(sum exp)
 *   ws    device workspace of at least attn_workspace_bytes(kv, n_q_heads, 1),
 *         16-byte aligned
 * Requires n_rows >= 1, n_q_heads a multiple of n_kv, 1 <= n_q_heads <= 4096,
 * d <= 1024 (FP8, TQ4) or d <= 512 (Q2K). */
kvq_status attn_decode_quant(const kvq_cache* kv, const float* q, int32_t n_q_heads,
                             float sm_scale, float* out, float* lse,
                             void* ws, size_t ws_bytes, void* stream);

/* One decode step of a KV8 cache that has just grown by one row: the step's
 * new latent row x_new is encoded into the cache's last row (n_rows - 1),
 * then the query attends every row, that one included.  The producer and the
 * consumer of [colibri #399] "Summary" / "Commits" item 1 and "Ready for
 * review" comment, as one call: the result, the written bytes and every error
 * are those of kv_encode_fp8(x_new, 1, d, codes + (n_rows-1) d,
 * scales + n_rows - 1) followed by attn_decode_quant(kv, q, ...).
 *   kv      FP8 cache, n_rows counting the new row (KVQ_ERR_UNSUPPORTED for
 *           other formats)
 *   x_new   f32 [d]        the new row
 *   codes   u8  [n_rows][d]   the cache's codes, the same buffer as
 *   scales  f32 [n_rows]      kv->codes / kv->scales (KVQ_ERR_SHAPE otherwise);
 *                             row n_rows - 1 is written, nothing else
 *   q, n_q_heads, sm_scale, out, lse, ws, ws_bytes, stream: as for
 *   attn_decode_quant (the same workspace size).
 * Where the decode runs per group of 16 heads on dense rows (d = 512, no rope
 * part, x_new 16-byte aligned), the decode launch itself encodes the row: the
 * workgroups whose chunk holds it encode it and take its codes from
 * registers, one of them writes it, and no workgroup reads it back from the
 * cache.  Otherwise the encoder runs first, then the decode. */
kvq_status attn_decode_append_fp8(const kvq_cache* kv, const float* x_new, uint8_t* codes,
                                  float* scales, const float* q, int32_t n_q_heads,
                                  float sm_scale, float* out, float* lse, void* ws,
                                  size_t ws_bytes, void* stream);

/* Chunked-prefill attention: S new query tokens at absolute positions
 * pos0 .. pos0+S-1 over a cache whose rows [pos0, pos0+S) were already
 * encoded (call kv_encode_* first, same stream).  Query s attends rows
 * t <= pos0 + s (causal).  [colibri #399] "Summary" (vectorized fp8 prefill).
 *   q    f32 [S][n_q_heads][d + d_rope];  out f32 [S][n_q_heads][d];
 *   lse  f32 [S][n_q_heads] or NULL
 *   ws   16-byte aligned, at least attn_workspace_bytes(kv, n_q_heads, S)
 * Requires pos0 >= 0, S >= 1, pos0 + S <= n_rows. */
kvq_status attn_prefill_quant(const kvq_cache* kv, const float* q, int32_t S,
                              int32_t n_q_heads, int64_t pos0, float sm_scale,
                              float* out, float* lse, void* ws, size_t ws_bytes,
                              void* stream);

/* Size of the device scratch attn_decode_quant_noalloc uses in place of a
 * caller workspace (one copy per GPU, held until the process ends). */
#define KVQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* attn_decode_quant without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and checks as
 * attn_decode_quant; the chunk partials go to a library-owned device array of
 * KVQ_NOALLOC_SCRATCH_BYTES per GPU instead of `ws`.  The call allocates and
 * frees nothing (the array is part of the library's code object).  Requests
 * whose attn_decode_quant workspace would exceed KVQ_NOALLOC_SCRATCH_BYTES
 * return KVQ_ERR_SCRATCH without enqueueing anything.  The matrix-core
 * decodes fit at any T: KV8 and TQ4 with d = 512 (any head count) need at
 * most 8.4 MB (about 256 chunks x 16 heads x 514 floats), q2k with d = 256
 * at most 2.1 MB.  All calls on one GPU share its array: calls that
 * may overlap on one GPU (several streams or host threads) race and must be
 * serialized by the caller.  The first call on a device looks the array's
 * address up (hipGetSymbolAddress) with that device current. */
kvq_status attn_decode_quant_noalloc(const kvq_cache* kv, const float* q, int32_t n_q_heads,
                                     float sm_scale, float* out, float* lse, void* stream);

/* Bytes of device workspace attn_decode_gather needs for a list of n_idx
 * entries (0 when the request is not supported, see attn_decode_gather). */
size_t attn_gather_workspace_bytes(const kvq_cache* kv, int32_t n_q_heads, int64_t n_idx);

/* One-token attention over a selected list of cached rows (top-k sparse
 * decode): the rows attended are idx[0], idx[1], ... of the cache, read by
 * absolute row index straight from the encoded cache.  [colibri #399]
 * "Commits" item 2 (the sparse-attention-aware gather) and the rebase
 * comment's item "1. DSA gather".  Scores, softmax and context as in
 * attn_decode_quant, over the listed rows only.
 *   idx   i32 [n_idx] device: absolute cache rows.  An entry outside
 *         [0, kv->n_rows) is padding and is skipped; a repeated entry is
 *         attended once per occurrence.  With no valid entry, out = 0 and
 *         lse = -inf.
 *   q     f32 [n_q_heads][d + d_rope];  out f32 [n_q_heads][d];
 *         lse f32 [n_q_heads] or NULL
 *   ws    16-byte aligned, at least attn_gather_workspace_bytes(kv,
 *         n_q_heads, n_idx)
 * Supported: FP8 and TQ4 latent caches with d = 512 and d_rope 0 or 64
 * (any n_q_heads >= 1), codes, scales, rope codes / scales and q 16-byte
 * aligned (KVQ_ERR_UNSUPPORTED otherwise);
 * 1 <= n_idx <= 2^31 - 1. */
kvq_status attn_decode_gather(const kvq_cache* kv, const int32_t* idx, int64_t n_idx,
                              const float* q, int32_t n_q_heads, float sm_scale,
                              float* out, float* lse, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * Helpers
 * ------------------------------------------------------------------------ */

/* Stored bytes per cached row for a format (KV8 d+4, TQ4 d/2+4, Q2K per cell
 * of n_kv heads: n_kv*(d/4 + d/16 + 18*d/32)), or 0 for an invalid request. */
size_t kvq_row_bytes(int32_t fmt, int32_t d, int32_t n_kv);

/* The codebook this library quantizes with: `levels` (4 or 16) Lloyd-Max
 * levels for N(0,1), rounded to fp16, ascending, written as f32 to host
 * memory `out`.  Returns KVQ_ERR_SHAPE for other level counts. */
kvq_status kvq_codebook(int32_t levels, float* out);

/* Human-readable status text (static storage). */
const char* kvq_status_str(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
