"""Plain CPU oracle for quantized-KV-cache attention (KV8 / TQ4 / q2k).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline leg
of the benchmark use it.  It shares no code, tables or constants with the HIP
library; the only thing both sides share is the seeded input generator in
`synth/`, which holds none of the method's arithmetic.

It is deliberately slow and literal: numpy float32 for every encoder step whose
rounding decides a stored byte (each numpy float32 add / multiply / divide /
sqrt is one IEEE-754 correctly rounded operation, there is no fused
multiply-add and every reduction order is written out), and float64 for the
attention, which is exactly softmax attention over the *decoded* cache.

Pages cited (titles abbreviated):
  [colibri #399]  "KV cache quantization: fp8 (KV8) + 4-bit TurboQuant (KV_TQ)
                   on CPU, CUDA, and Metal"
  [colibri #553]  "CPU: KV cache quantization - KV8 (fp8 e4m3) + KV_TQ
                   (rotated-int4 / PolarQuant)"
  [Strata #2318]  "KV cache: FP16 sliding window + attention sinks, and an
                   optional 2-bit K / 4-bit V cache scheme (--kv q2k)"
External published definitions used where the pages are silent:
  SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014) for the rotation signs; Lloyd (1957) / Max (1960)
  for the Gaussian minimum-MSE quantizer levels.

Where the pages leave a step open, the reading taken is the one listed in the
design notes of this repository; each function says which reading it takes.
Parity status: every function below is pinned by a `-m "not gpu"` test
(tests/test_oracle_*.py) against page-printed values, closed forms,
invariants, brute force or an independent library routine.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import ndtr

F32 = np.float32
M64 = (1 << 64) - 1

# --------------------------------------------------------------------------
# fp8 e4m3 (KV8)
# --------------------------------------------------------------------------


def e4m3_table() -> np.ndarray:
    """Value of every fp8 e4m3 byte, float64 [256].

    [colibri #399], rebase comment, item "3. HIP portability": normals are
    (1+M/8)*2^(E-7), denormals M*2^-9, and S.1111.111 reads back as 0.
    """
    out = np.empty(256, np.float64)
    for b in range(256):
        s, e, m = b >> 7, (b >> 3) & 15, b & 7
        if e == 15 and m == 7:
            v = 0.0
        elif e == 0:
            v = m * 2.0 ** -9
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[b] = -v if (s and v != 0.0) else v
    return out


def e4m3_rne_magnitude(a: np.ndarray) -> np.ndarray:
    """Round |v| (float32, finite, >= 0) to the nearest e4m3 magnitude code.

    Round-to-nearest-even on the 3-bit mantissa, subnormals below 2^-6, and
    saturation to the largest finite value 448 (code 0x7E) for anything at or
    above it.  [colibri #399] "Commits", item 1: the encoder rounds RNE; the
    largest e4m3 value is the 448 of the amax/448 scale.
    """
    a64 = np.asarray(a, np.float32).astype(np.float64)   # exact widening
    codes = np.zeros(a64.shape, np.int64)
    sub = a64 < 2.0 ** -6
    # subnormal range: value = M * 2^-9, M = 0..7 (M = 8 is the first normal)
    m_sub = np.rint(np.where(sub, a64, 0.0) * 512.0).astype(np.int64)   # exact scaling; rint = half-even
    codes = np.where(sub, m_sub, codes)
    # normal range: a = f * 2^k with f in [0.5, 1)  =>  exponent e = k - 1
    _, k = np.frexp(np.where(sub, 1.0, a64))
    e = k.astype(np.int64) - 1
    mm = np.rint(np.ldexp(np.where(sub, 1.0, a64), (3 - e).astype(np.int32))).astype(np.int64)
    carry = mm == 16                                       # rounded up to the next binade
    e = np.where(carry, e + 1, e)
    mm = np.where(carry, 8, mm)
    c_norm = ((e + 7) << 3) | (mm - 8)
    codes = np.where(sub, codes, c_norm)
    codes = np.where(a64 >= 448.0, 0x7E, codes)           # saturate
    codes = np.minimum(codes, 0x7E)
    return codes.astype(np.uint8)


def kv8_encode(x: np.ndarray):
    """KV8 row encoder: fp8 e4m3 codes + one float32 scale per row.

    [colibri #399] "Summary" and "Commits" item 1 (fp8 e4m3 + per-row scale,
    RNE, scale = amax/448); [colibri #553] "What's in it" (the per-row scale
    factors out of the sums).  Reading: scale = fl32(amax / 448); each element
    is divided by the stored scale in float32 and rounded RNE; the sign bit is
    the sign bit of that quotient; a row whose scale is 0 stores all-zero
    codes and scale 0.
    Returns (codes uint8 [n, d], scales float32 [n]).
    """
    x = np.ascontiguousarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1)                      # max is order-free
    scale = amax / F32(448.0)                             # one IEEE f32 divide
    live = scale > 0
    div = np.where(live, scale, F32(1.0)).astype(np.float32)
    v = x / div[:, None]                                  # IEEE f32 divide per element
    mag = e4m3_rne_magnitude(np.abs(v))
    sign = (np.signbit(v).astype(np.uint8) << 7).astype(np.uint8)
    codes = np.where(live[:, None], mag | sign, 0).astype(np.uint8)
    return codes, np.where(live, scale, F32(0.0)).astype(np.float32)


def kv8_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_hat = e4m3(code) * scale, exact in float64 [colibri #553] "What's in it"."""
    lut = e4m3_table()
    return lut[np.asarray(codes)] * np.asarray(scales, np.float64)[..., None]


# --------------------------------------------------------------------------
# Rotation: seeded random signs + fast Walsh-Hadamard transform
# --------------------------------------------------------------------------


def splitmix64(seed: int, count: int) -> list[int]:
    """First `count` outputs of SplitMix64 started from state `seed`.

    Published definition (Steele, Lea, Flood 2014): state += 0x9E3779B97F4A7C15;
    z = state; z = (z ^ z>>30) * 0xBF58476D1CE4E5B9; z = (z ^ z>>27) *
    0x94D049BB133111EB; output z ^ z>>31 (all mod 2^64).
    """
    state = seed & M64
    out = []
    for _ in range(count):
        state = (state + 0x9E3779B97F4A7C15) & M64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
        out.append(z ^ (z >> 31))
    return out


def rotation_signs(seed: int, n: int) -> np.ndarray:
    """The +-1 diagonal D of the randomized Hadamard rotation, float32 [n].

    [colibri #399] "Why rotated-int4 for the 4-bit tier" (a randomized-Hadamard
    rotation).  The pages do not say how the signs are drawn; reading: sign i is
    -1 exactly when bit (i mod 64) of SplitMix64 output number floor(i/64) is 1.
    """
    words = splitmix64(seed, (n + 63) // 64)
    bits = np.array([(words[i // 64] >> (i % 64)) & 1 for i in range(n)], np.int64)
    return np.where(bits == 1, -1.0, 1.0).astype(np.float32)


def _fwht(v: np.ndarray, dtype) -> np.ndarray:
    v = np.array(v, dtype=dtype, copy=True)
    n = v.shape[-1]
    lead = v.shape[:-1]
    h = 1
    while h < n:
        w = v.reshape(lead + (n // (2 * h), 2, h))
        a = w[..., 0, :].copy()
        b = w[..., 1, :].copy()
        w[..., 0, :] = a + b
        w[..., 1, :] = a - b
        h *= 2
    return v


def fwht_f32(v: np.ndarray) -> np.ndarray:
    """Unnormalised radix-2 fast Walsh-Hadamard transform in float32.

    [colibri #553] rebase comment on non-power-of-two rows (both codecs rotate
    through a radix-2 FWHT).  Reading: stages h = 1, 2, 4, ..., n/2 in that
    order; each pair (i, i+h) with bit h of i clear becomes (a+b, a-b), each a
    single f32 rounding.  Works on the last axis, which must be a power of 2.
    """
    return _fwht(v, np.float32)


def fwht_f64(v: np.ndarray) -> np.ndarray:
    """The same transform in float64 (used only on the decode side)."""
    return _fwht(v, np.float64)


# --------------------------------------------------------------------------
# Lloyd-Max codebooks for N(0,1)
# --------------------------------------------------------------------------

_CB_CACHE: dict[int, tuple[np.ndarray, float]] = {}


def lloyd_max_gaussian(levels: int, tol: float = 1e-15, max_iter: int = 200000):
    """Minimum-MSE scalar quantizer levels for N(0,1) (Lloyd 1957 / Max 1960).

    [colibri #399] "Why rotated-int4 for the 4-bit tier": a fixed 16-level
    Lloyd-Max codebook, N(0,1)-optimal.  [Strata #2318] "Why per-channel K and
    per-token V": a 4-level Lloyd-Max codebook for K.  Iterates the two
    optimality conditions in float64: boundaries are midpoints of adjacent
    levels; each level is the conditional mean of N(0,1) on its cell,
    (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  Returns (levels f64 ascending,
    mean squared error).
    """
    c = np.array([ndtr_inv_mid(levels, k) for k in range(levels)], np.float64)
    for _ in range(max_iter):
        b = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
        pdf = np.where(np.isfinite(b), np.exp(-0.5 * np.where(np.isfinite(b), b, 0.0) ** 2), 0.0) / math.sqrt(2 * math.pi)
        prob = ndtr(b[1:]) - ndtr(b[:-1])
        c_new = (pdf[:-1] - pdf[1:]) / prob
        done = np.max(np.abs(c_new - c)) < tol
        c = c_new
        if done:
            break
    b = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    return c, gaussian_quantizer_mse(c, b)


def ndtr_inv_mid(levels: int, k: int) -> float:
    """Starting point: the N(0,1) quantile at the centre of equal-mass cell k."""
    from scipy.special import ndtri
    return float(ndtri((k + 0.5) / levels))


def gaussian_quantizer_mse(c: np.ndarray, b: np.ndarray) -> float:
    """E[(Z - Q(Z))^2] for Z ~ N(0,1), levels c, cell boundaries b (closed form)."""
    phi = lambda z: 0.0 if not np.isfinite(z) else math.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)
    zphi = lambda z: 0.0 if not np.isfinite(z) else z * phi(z)
    total = 0.0
    for k in range(len(c)):
        a, bb = b[k], b[k + 1]
        p = float(ndtr(bb) - ndtr(a))
        m1 = phi(a) - phi(bb)                      # int z phi
        m2 = p + zphi(a) - zphi(bb)                # int z^2 phi
        total += m2 - 2 * c[k] * m1 + c[k] ** 2 * p
    return total


def codebook_f16(levels: int) -> np.ndarray:
    """The stored codebook: Lloyd-Max levels rounded to the nearest float16,
    held as float32 (reading: f16-representable levels, so codebook operands
    are exact in half precision)."""
    if levels not in _CB_CACHE:
        _CB_CACHE[levels] = lloyd_max_gaussian(levels)
    c, _ = _CB_CACHE[levels]
    return c.astype(np.float16).astype(np.float32)


def codebook_thresholds(levels: int) -> np.ndarray:
    """Decision thresholds tau_k = (c_k + c_{k+1}) / 2 of the f16 codebook
    (exact in float32: the sum of two f16 values fits in 24 bits)."""
    c = codebook_f16(levels)
    return ((c[:-1] + c[1:]) / F32(2.0)).astype(np.float32)


# --------------------------------------------------------------------------
# TQ4: rotated-int4 codec
# --------------------------------------------------------------------------


def is_pow2(n: int) -> bool:
    return n >= 2 and (n & (n - 1)) == 0


def tq4_radius(x: np.ndarray) -> np.ndarray:
    """Row radius ||x||_2 in float32 with a fixed pairwise tree.

    [colibri #399] "Why rotated-int4 for the 4-bit tier": the rotation keeps
    the radius, so one per-row scale survives.  Reading: p_i = fl32(x_i*x_i);
    for h = n/2, n/4, ..., 1: p_i = fl32(p_i + p_{i+h}) for i < h; r = sqrtf(p_0).
    """
    x = np.asarray(x, np.float32)
    with np.errstate(over="ignore"):          # rows near the float32 limit: r = inf, as in float32
        p = x * x
        h = x.shape[-1] // 2
        while h >= 1:
            p = p[..., :h] + p[..., h:2 * h]
            h //= 2
    return np.sqrt(p[..., 0]).astype(np.float32)


def tq4_encode(x: np.ndarray, seed: int):
    """Rotated-int4 row encoder: packed nibbles + float32 radius per row.

    [colibri #399] "Why rotated-int4 for the 4-bit tier" (randomized-Hadamard
    rotation, fixed 16-level N(0,1) Lloyd-Max codebook scaled by radius/sqrt(n),
    full reconstruction) and [colibri #553] "What's in it" (the radius rides
    the per-row scale).  Steps: r = radius; y = FWHT(D*x) (unnormalised, so
    mean(y_i^2) = r^2 and y_i / r is matched to the N(0,1) book); the level of
    y_i is the number of thresholds fl32(tau_k * r) strictly below y_i (ties
    go to the lower level); element 2j goes to the low nibble of byte j.  A
    zero radius stores all-zero bytes (the pages' inert row).
    Returns (packed uint8 [n_rows, n/2], radius float32 [n_rows]).
    """
    x = np.ascontiguousarray(x, np.float32)
    n = x.shape[1]
    if not is_pow2(n):
        raise ValueError("TQ4 needs a power-of-two row width")
    r = tq4_radius(x)
    y = fwht_f32(x * rotation_signs(seed, n)[None, :])
    tau = codebook_thresholds(16)
    idx = np.zeros(y.shape, np.int64)
    for k in range(15):
        with np.errstate(invalid="ignore", over="ignore"):   # r = inf: the middle threshold is NaN
            thr = (tau[k] * r).astype(np.float32)
        idx += (y > thr[:, None])
    idx[r == 0] = 0
    packed = (idx[:, 0::2] | (idx[:, 1::2] << 4)).astype(np.uint8)
    return packed, r


def tq4_unpack(packed: np.ndarray) -> np.ndarray:
    """Nibble indices [rows, n] from packed bytes [rows, n/2]."""
    p = np.asarray(packed, np.int64)
    idx = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.int64)
    idx[..., 0::2] = p & 15
    idx[..., 1::2] = p >> 4
    return idx


def tq4_decode(packed: np.ndarray, radius: np.ndarray, seed: int) -> np.ndarray:
    """x_hat = (r/n) * D * H c[idx], in float64.

    Inverse of the rotation y = H D x: (H D)^-1 = D H / n.  [colibri #399]
    "Why rotated-int4 for the 4-bit tier" (full reconstruction).
    """
    idx = tq4_unpack(packed)
    n = idx.shape[-1]
    c = codebook_f16(16).astype(np.float64)
    y = fwht_f64(c[idx])
    d = rotation_signs(seed, n).astype(np.float64)
    return y * d[None, :] * (np.asarray(radius, np.float64)[:, None] / n)


# --------------------------------------------------------------------------
# q2k: 2-bit per-channel K + q4_0 per-token V + fp16 sink/window overlay
# --------------------------------------------------------------------------

Q2K_GROUP = 32


def f16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit pattern, round to nearest even."""
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def f16_value(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def q2k_encode_k(k: np.ndarray, k_gain: float):
    """2-bit per-channel K ("block_q2c_0") with the K reconstruction gain.

    [Strata #2318] "Summary" item 3 and "Why per-channel K and per-token V":
    one fp16 scale per dimension per 32-cell group, a 4-level Lloyd-Max
    codebook; the stored scale is B times the rule's while the codes are chosen
    against the un-gained scale.  Readings: the rule is the RMS over the 32
    cells of the group, sum of squares accumulated in cell order in float32;
    s = sqrtf(ss / 32); level = number of thresholds fl32(tau_m * s) strictly
    below the value; stored scale = f16_RNE(fl32(B * s)); a zero s stores
    codes 0 and scale 0.  Byte q of (group, head, channel) holds cells
    4q..4q+3, cell j in bits 2*(j mod 4).
    k: float32 [T, n_kv, d], T a multiple of 32.
    Returns (codes uint8 [T/32, n_kv, d, 8], scale bits uint16 [T/32, n_kv, d]).
    """
    k = np.ascontiguousarray(k, np.float32)
    T, n_kv, d = k.shape
    G = T // Q2K_GROUP
    kg = k.reshape(G, Q2K_GROUP, n_kv, d)
    ss = np.zeros((G, n_kv, d), np.float32)
    for j in range(Q2K_GROUP):                     # sequential, cell order
        ss = ss + kg[:, j] * kg[:, j]
    s_rule = np.sqrt(ss / F32(32.0)).astype(np.float32)
    tau = codebook_thresholds(4)
    codes = np.zeros((G, Q2K_GROUP, n_kv, d), np.int64)
    for m in range(3):
        thr = (tau[m] * s_rule).astype(np.float32)
        codes += kg > thr[:, None, :, :]
    codes = np.where((s_rule == 0)[:, None, :, :], 0, codes)
    c = codes.transpose(0, 2, 3, 1).reshape(G, n_kv, d, 8, 4)      # [G,h,c,q,i]
    packed = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
    stored = f16_bits((F32(k_gain) * s_rule).astype(np.float32))
    return packed, stored


def q2k_encode_v(v: np.ndarray):
    """q4_0 V blocks: 32 values per block, 18 bytes (fp16 d, then 16 bytes).

    [Strata #2318] "Why per-channel K and per-token V" (V reuses q4_0, per-token
    blocks); the block layout and decode rule are the ones the third-party
    INT8-overlay review diff on that page reads back: d is the first two
    bytes (little-endian fp16), element j < 16 is the low nibble of byte j,
    element j >= 16 the high nibble of byte j-16, value (code - 8) * d.  The
    page gives only the decode; reading for the encode: d = f16_RNE(fl32(amax
    / 7)); code = clamp(rint(fl32(x / d)) + 8, 0, 15); a block with d = 0
    stores code 8 everywhere.
    v: float32 [T, n_kv, d].  Returns uint8 [T, n_kv, d/32, 18].
    """
    v = np.ascontiguousarray(v, np.float32)
    T, n_kv, d = v.shape
    vb = v.reshape(T, n_kv, d // 32, 32)
    amax = np.max(np.abs(vb), axis=-1)
    d16 = f16_bits((amax / F32(7.0)).astype(np.float32))
    df = d16.view(np.float16).astype(np.float32)
    zero = df == 0
    q = np.rint(vb / np.where(zero, F32(1.0), df)[..., None]).astype(np.float32)
    code = np.clip(q + F32(8.0), 0, 15).astype(np.int64)
    code = np.where(zero[..., None], 8, code)
    out = np.zeros((T, n_kv, d // 32, 18), np.uint8)
    out[..., 0] = (d16 & 0xFF).astype(np.uint8)
    out[..., 1] = (d16 >> 8).astype(np.uint8)
    out[..., 2:] = (code[..., :16] | (code[..., 16:] << 4)).astype(np.uint8)
    return out


def overlay_slot(t: int, n_sink: int, n_window: int, n_slack: int = 0) -> int:
    """Overlay slot of cell t: a sink keeps slot t; any later cell has the
    ring slot n_sink + (t - n_sink) mod (n_window + n_slack).

    [Strata #2318] "Summary" item 1: an fp16 overlay over the first S cells
    (sinks) and the most recent N cells, sized S + N + 16 slack slots.
    Reading: the window is a ring of N + slack slots, so a cell's slot is
    fixed when it is written and never depends on how many cells follow;
    the slack lets up to `n_slack` cells be written ahead (a speculative
    window) without overwriting a cell that is still in the window."""
    if t < n_sink:
        return t
    return n_sink + (t - n_sink) % (n_window + n_slack)


def overlay_live(t: int, T: int, n_sink: int, n_window: int) -> bool:
    """Cell t of a cache of T cells reads its fp16 copy: a sink (t < S) or one
    of the last N cells."""
    return 0 <= t < T and (t < n_sink or t >= T - n_window)


def overlay_slot_cells(T: int, n_sink: int, n_window: int, n_slack: int = 0) -> np.ndarray:
    """Cell held by each of the n_sink + n_window + n_slack slots for the live
    cells of a cache of T cells (-1: the slot holds no live cell)."""
    cells = np.full(n_sink + n_window + n_slack, -1, np.int64)
    for t in range(max(0, T - n_window - n_sink), T):
        if overlay_live(t, T, n_sink, n_window):
            cells[overlay_slot(t, n_sink, n_window, n_slack)] = t
    for t in range(min(n_sink, T)):
        cells[t] = t
    return cells


def q2k_overlay_write(k_ovl, v_ovl, k: np.ndarray, v: np.ndarray, c0: int, c1: int,
                      n_sink: int, n_window: int, n_slack: int):
    """Batch overlay writer for appended cells [c0, c1) (k, v hold every cell
    up to c1): sinks go to their slots, and of the other cells only the last
    n_window + n_slack of the cache (the ones a one-cell-at-a-time writer
    would leave in the ring) are written, so every writer ends with the same
    slots.  [Strata #2318] "Review fixes" (writers single / speculative
    multi-step / batch agree on every live cell).  In place."""
    R = n_window + n_slack
    for c in range(c0, c1):
        if c < n_sink or (R > 0 and c >= c1 - R):
            sl = overlay_slot(c, n_sink, n_window, n_slack)
            k_ovl[sl] = f16_bits(np.asarray(k[c], np.float32))
            v_ovl[sl] = f16_bits(np.asarray(v[c], np.float32))


def q2k_encode(k: np.ndarray, v: np.ndarray, k_gain: float, n_sink: int, n_window: int,
               n_slack: int = 0):
    """Whole q2k cache for cells [0, T): K codes + K scales, V blocks and the
    fp16 overlay (k_ovl, v_ovl [n_sink + n_window + n_slack, n_kv, d] uint16;
    slots no cell was written to are zero).  [Strata #2318] "Summary" items
    1-3."""
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    T, n_kv, d = k.shape
    kc, ks = q2k_encode_k(k, k_gain)
    vb = q2k_encode_v(v)
    k_ovl = np.zeros((n_sink + n_window + n_slack, n_kv, d), np.uint16)
    v_ovl = np.zeros_like(k_ovl)
    q2k_overlay_write(k_ovl, v_ovl, k, v, 0, T, n_sink, n_window, n_slack)
    return kc, ks, vb, k_ovl, v_ovl


def q2k_group_scale(ss: np.ndarray, n: int, prev) -> np.ndarray:
    """Un-gained K scale of a 32-cell group holding n cells, from the f32 sum
    of squares ss of those cells (per head and channel).

    [Strata #2318] "Review fixes" and "Attention error under the engine's
    append patterns": a whole group takes the RMS rule sqrtf(ss / 32); a
    partial group is shrunk toward the previous group's scale prev, standing
    in for the cells not yet written: sqrtf((ss + (32 - n) prev^2) / 32).
    Reading: the first group (no previous one) takes the RMS of the cells
    present, sqrtf(ss / n).  f32 order: prev*prev, times (32 - n), plus ss,
    divided by 32."""
    ss = np.asarray(ss, np.float32)
    if n == Q2K_GROUP:
        return np.sqrt(ss / F32(32.0)).astype(np.float32)
    if prev is None:
        return np.sqrt(ss / F32(n)).astype(np.float32)
    prev = np.asarray(prev, np.float32)
    fill = (F32(Q2K_GROUP - n) * (prev * prev)).astype(np.float32)
    return np.sqrt((ss + fill).astype(np.float32) / F32(32.0)).astype(np.float32)


def q2k_append(state: dict, k: np.ndarray, v: np.ndarray, n_prev: int, n_new: int, k_gain: float,
               n_sink: int, n_window: int, n_slack: int) -> dict:
    """Append cells [n_prev, n_prev + n_new) to a q2k cache (a new state; the
    input is not modified).

    k, v: float32 [>= n_prev + n_new, n_kv, d], every cell so far (only the
    groups this call touches are read).  state: k_codes [G, n_kv, d, 8],
    k_scale [G, n_kv, d] (uint16 bits), v_blocks [>= cells, n_kv, d/32, 18],
    k_ovl / v_ovl [n_sink + n_window + n_slack, n_kv, d].
    Readings ([Strata #2318] "Review fixes", "Attention error under the
    engine's append patterns"): every group this call touches is requantized
    from all of its cells present so far -- scale by q2k_group_scale, codes
    of those cells against the un-gained scale, stored scale f16(B * s),
    absent cells code 0 -- so a group completed over several calls ends as
    the one-shot encoder would leave it; prev is the previous group's stored
    scale divided by B (in f32), which the same rule reproduces whether that
    group was completed in this call or an earlier one (two-call and
    one-call appends store the same scale).  V blocks are per cell (q4_0 of
    the new cells); the overlay gets the batch writer's slots."""
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    st = {key: np.array(val, copy=True) for key, val in state.items()}
    n_end = n_prev + n_new
    _, n_kv, d = k.shape
    tau = codebook_thresholds(4)
    B = F32(k_gain)
    for g in range(n_prev // Q2K_GROUP, (n_end + Q2K_GROUP - 1) // Q2K_GROUP):
        c0 = g * Q2K_GROUP
        n = min(Q2K_GROUP, n_end - c0)
        cells = k[c0:c0 + n]                                   # [n, n_kv, d]
        ss = np.zeros((n_kv, d), np.float32)
        for j in range(n):                                     # cell order
            ss = (ss + cells[j] * cells[j]).astype(np.float32)
        prev = None
        if g > 0:
            prev = (f16_value(st["k_scale"][g - 1]).astype(np.float32) / B).astype(np.float32)
        s_rule = q2k_group_scale(ss, n, prev)
        codes = np.zeros((Q2K_GROUP, n_kv, d), np.int64)
        for m in range(3):
            thr = (tau[m] * s_rule).astype(np.float32)
            codes[:n] += cells > thr[None]
        codes[:, s_rule == 0] = 0
        c = codes.transpose(1, 2, 0).reshape(n_kv, d, 8, 4)
        st["k_codes"][g] = (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)
        st["k_scale"][g] = f16_bits((B * s_rule).astype(np.float32))
    st["v_blocks"][n_prev:n_end] = q2k_encode_v(v[n_prev:n_end])
    q2k_overlay_write(st["k_ovl"], st["v_ovl"], k, v, n_prev, n_end, n_sink, n_window, n_slack)
    return st


def q2k_empty_state(cap_cells: int, n_kv: int, d: int, n_sink: int, n_window: int, n_slack: int) -> dict:
    """Zeroed q2k buffers for up to cap_cells cells (appends fill them)."""
    G = (cap_cells + Q2K_GROUP - 1) // Q2K_GROUP
    n_ovl = n_sink + n_window + n_slack
    return {"k_codes": np.zeros((G, n_kv, d, 8), np.uint8),
            "k_scale": np.zeros((G, n_kv, d), np.uint16),
            "v_blocks": np.zeros((G * Q2K_GROUP, n_kv, d // 32, 18), np.uint8),
            "k_ovl": np.zeros((n_ovl, n_kv, d), np.uint16),
            "v_ovl": np.zeros((n_ovl, n_kv, d), np.uint16)}


def q2k_decode(k_codes, k_scale, v_blocks, k_ovl, v_ovl, n_sink: int, n_window: int,
               n_slack: int = 0, T: int | None = None):
    """Decoded K, V (float64 [T, n_kv, d]) as the attention reads them, for a
    cache of T cells (default: every cell of the groups given).

    Bulk K: l[code] * scale (4-level f16 book); bulk V: (code - 8) * d;
    overlay cells (sinks and the last n_window cells, ring slots) read the
    fp16 copies instead [Strata #2318] "Summary" item 1 and "Measurements"
    (sink and window cells read bit-exactly)."""
    G, n_kv, d, _ = k_codes.shape
    if T is None:
        T = G * Q2K_GROUP
    lv = codebook_f16(4).astype(np.float64)
    b = np.asarray(k_codes, np.int64)
    codes = np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=-1)   # [G,h,c,q,i]
    codes = codes.reshape(G, n_kv, d, Q2K_GROUP).transpose(0, 3, 1, 2)  # [G,j,h,c]
    K = lv[codes] * f16_value(k_scale)[:, None, :, :]
    K = K.reshape(G * Q2K_GROUP, n_kv, d)[:T]
    vb = np.asarray(v_blocks, np.int64)[:T]
    dv = f16_value((vb[..., 0] | (vb[..., 1] << 8)).astype(np.uint16))   # [T,h,nb]
    nib = vb[..., 2:]
    code = np.concatenate([nib & 15, nib >> 4], axis=-1)                  # [T,h,nb,32]
    V = ((code - 8) * dv[..., None]).reshape(T, n_kv, d)
    cells = overlay_slot_cells(T, n_sink, n_window, n_slack)
    live = cells >= 0
    if k_ovl is not None and live.any():
        K[cells[live]] = f16_value(np.asarray(k_ovl)[live])
        V[cells[live]] = f16_value(np.asarray(v_ovl)[live])
    return K, V


# --------------------------------------------------------------------------
# Attention over decoded rows (float64)
# --------------------------------------------------------------------------


def attention_decode(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float, heads=None,
                     dtype=np.float64):
    """Single-token attention, float64.

    out_h = sum_t w_t V_t / sum_t w_t with w_t = exp(s_t - max s), s_t =
    sm_scale * q_h . K_t, and lse_h = max s + ln sum w.  [colibri #399]
    "Ready for review" comment (scores against the encoded rows, then context);
    the MLA latent row is both key and value ("Why rotated-int4 ...").
    q: [Hq, d]; K, V: [T, n_kv, d] (or [T, d] for one shared latent head).
    Query head h reads KV head h // (Hq / n_kv) (contiguous grouping).
    Returns (out float64 [len(heads), d], lse float64 [len(heads)]).
    `dtype` float32 evaluates the same formulas in single precision: the tests
    use that twin only to size what plain f32 rounding does to each row.
    """
    q = np.asarray(q, dtype)
    K = np.asarray(K, dtype)
    V = np.asarray(V, dtype)
    if K.ndim == 2:
        K = K[:, None, :]
        V = V[:, None, :]
    Hq = q.shape[0]
    n_kv = K.shape[1]
    group = Hq // n_kv
    heads = range(Hq) if heads is None else heads
    outs, lses = [], []
    for h in heads:
        g = h // group
        s = (K[:, g, :] @ q[h]) * dtype(sm_scale)
        m = np.max(s)
        w = np.exp(s - m)
        l = np.sum(w)
        outs.append((w @ V[:, g, :]) / l)
        lses.append(float(m) + math.log(float(l)))
    return np.array(outs), np.array(lses)


def attention_decode_gather(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx, sm_scale: float,
                            dtype=np.float64):
    """Single-token attention over a selected list of cached rows, float64.

    The rows attended are K[idx[i]], V[idx[i]] for i in list order: an
    absolute-index gather of the selected (top-k) rows, [colibri #399]
    "Commits" item 2 (the sparse-attention-aware gather) and the rebase comment's item "1.
    DSA gather" (the fp8 cache's absolute-index gather of the selection).
    Reading (the pages are silent on padding): an index outside [0, T) is a
    padding entry and is skipped; a repeated index is attended once per
    occurrence.  With no valid index the output is 0 and lse is -inf.
    Returns (out float64 [Hq, d], lse float64 [Hq]).
    """
    T = np.asarray(K).shape[0]
    rows = [int(i) for i in np.asarray(idx).reshape(-1) if 0 <= int(i) < T]
    Hq, d = np.asarray(q).shape
    if not rows:
        return np.zeros((Hq, d), np.float64), np.full((Hq,), -np.inf)
    Kg = np.asarray(K)[rows]
    Vg = np.asarray(V)[rows]
    return attention_decode(q, Kg, Vg, sm_scale, dtype=dtype)


def attention_prefill(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float, pos0: int,
                      rows=None, dtype=np.float64):
    """Causal chunked-prefill attention, float64: query s (absolute position
    pos0 + s) attends cached rows t <= pos0 + s.
    q: [S, Hq, d]; K, V as in attention_decode.  `rows` is an optional list of
    (s, h) pairs to compute (all pairs by default).
    Returns (out float64 [n_pairs, d], lse [n_pairs]) in the order of `rows`.
    `dtype`: as in attention_decode.
    """
    q = np.asarray(q, dtype)
    K = np.asarray(K, dtype)
    V = np.asarray(V, dtype)
    if K.ndim == 2:
        K = K[:, None, :]
        V = V[:, None, :]
    S, Hq, _ = q.shape
    group = Hq // K.shape[1]
    if rows is None:
        # every pair: the heads of one KV head and one token at once (the
        # same formulas, a matrix product over the heads in place of a
        # matrix-vector product per head)
        outs = np.empty((S, Hq, V.shape[2]), dtype)
        lses = np.empty((S, Hq))
        for s in range(S):
            lim = pos0 + s + 1
            for g in range(K.shape[1]):
                hs = slice(g * group, (g + 1) * group)
                sc = (K[:lim, g, :] @ q[s, hs].T) * dtype(sm_scale)     # [lim, group]
                m = np.max(sc, axis=0)
                w = np.exp(sc - m)
                l = np.sum(w, axis=0)
                outs[s, hs] = (w.T @ V[:lim, g, :]) / l[:, None]
                lses[s, hs] = m.astype(np.float64) + np.log(l.astype(np.float64))
        return outs.reshape(S * Hq, -1), lses.reshape(-1)
    outs, lses = [], []
    for s, h in rows:
        g = h // group
        lim = pos0 + s + 1
        sc = (K[:lim, g, :] @ q[s, h]) * dtype(sm_scale)
        m = np.max(sc)
        w = np.exp(sc - m)
        l = np.sum(w)
        outs.append((w @ V[:lim, g, :]) / l)
        lses.append(float(m) + math.log(float(l)))
    return np.array(outs), np.array(lses)


def attention_decode_rope(q: np.ndarray, K_lat: np.ndarray, K_rope: np.ndarray, sm_scale: float,
                          dtype=np.float64):
    """Single-token MLA attention whose key is the latent row followed by its
    rope row, float64.

    s_t = sm_scale * (q_lat . K_lat[t] + q_rope . K_rope[t]);
    out_h = sum_t w_t K_lat[t] / sum_t w_t, w_t = exp(s_t - max s); lse as in
    attention_decode.  The value is the latent part alone.  [colibri #553]
    rebase comment, item 1: a cached MLA row has a kv_lora part and a qk_rope
    part (512 and 64 wide on the pages' model), and each part is quantized on
    its own (TQ4 rotates each, so both widths must be powers of two).
    q: [Hq, d + d_rope], latent part first; K_lat [T, d]; K_rope [T, d_rope].
    Returns (out float64 [Hq, d], lse float64 [Hq]).  `dtype`: as in
    attention_decode.
    """
    q = np.asarray(q, dtype)
    Kl = np.asarray(K_lat, dtype)
    Kr = np.asarray(K_rope, dtype)
    d = Kl.shape[1]
    outs, lses = [], []
    for h in range(q.shape[0]):
        s = (Kl @ q[h, :d] + Kr @ q[h, d:]) * dtype(sm_scale)
        m = np.max(s)
        w = np.exp(s - m)
        l = np.sum(w)
        outs.append((w @ Kl) / l)
        lses.append(float(m) + math.log(float(l)))
    return np.array(outs), np.array(lses)


def attention_prefill_rope(q: np.ndarray, K_lat: np.ndarray, K_rope: np.ndarray, sm_scale: float,
                           pos0: int, rows=None, dtype=np.float64):
    """Causal chunked prefill with the latent + rope key of
    attention_decode_rope: query s (position pos0 + s) attends rows
    t <= pos0 + s.  q: [S, Hq, d + d_rope].  `rows`: optional (s, h) pairs.
    Returns (out float64 [n_pairs, d], lse [n_pairs]) in the order of `rows`.
    `dtype`: as in attention_decode."""
    q = np.asarray(q, dtype)
    Kl = np.asarray(K_lat, dtype)
    Kr = np.asarray(K_rope, dtype)
    S, Hq, _ = q.shape
    d = Kl.shape[1]
    if rows is None:
        rows = [(s, h) for s in range(S) for h in range(Hq)]
    outs, lses = [], []
    for s, h in rows:
        lim = pos0 + s + 1
        sc = (Kl[:lim] @ q[s, h, :d] + Kr[:lim] @ q[s, h, d:]) * dtype(sm_scale)
        m = np.max(sc)
        w = np.exp(sc - m)
        l = np.sum(w)
        outs.append((w @ Kl[:lim]) / l)
        lses.append(float(m) + math.log(float(l)))
    return np.array(outs), np.array(lses)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_2 / ||ref||_2 over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))


# --------------------------------------------------------------------------
# Byte accounting
# --------------------------------------------------------------------------


def row_bytes(fmt: str, d: int, n_kv: int = 1) -> float:
    """Stored bytes per cached row (KV8, TQ4: one latent row; q2k: one cell of
    n_kv heads).  [colibri #399] "Summary" (~3.9x / ~7.8x less than f32);
    [Strata #2318] "Memory" (448 B per cell at 2 heads x 256)."""
    if fmt == "fp8":
        return d + 4
    if fmt == "tq4":
        return d // 2 + 4
    if fmt == "q2k":
        k = n_kv * d * 2 / 8 + n_kv * d * 2 / 32        # 2-bit codes + fp16 scale per 32 cells
        v = n_kv * (d // 32) * 18                        # q4_0 blocks
        return k + v
    raise ValueError(fmt)
