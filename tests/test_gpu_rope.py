"""GPU attention over an MLA key with a rope part (key = latent | rope, value =
latent) vs the float64 oracle's attention_decode_rope / attention_prefill_rope.

Both parts are encoded on the GPU by the format's encoder (the rope rows at
their own width, TQ4 with their own seed); the bytes are checked equal to the
oracle's encoding, and the oracle decodes those bytes.  Output within 1e-5
relative L2, lse within 1e-5 relative error.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import kvq_oracle as o
from tests._gpu import check_attention, reference, assert_bytes_equal, dev, host, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_kv_cache_e4m3_amd as kq

TOL = 1e-5
ROPE_SEED = 0x0123456789ABCDEF


def _check(out, lse, ref_out, ref_lse, what, twin):
    check_attention(out, lse, ref_out, ref_lse, what, TOL, twin)


def _inputs(T, H, d, dr, seed, rope_gain=3.0):
    g = np.random.default_rng(seed)
    xl = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    xr = (g.standard_normal((T, dr)) * rope_gain).astype(np.float32)
    q = g.standard_normal((H, d + dr)).astype(np.float32)
    return xl, xr, q


def _cache(fmt, xl, xr, seed=777):
    """GPU cache with a rope part, and the oracle's decoded latent / rope rows."""
    if fmt == "fp8":
        c, s = kq.kv_encode_fp8(dev(xl))
        rc, rs = kq.kv_encode_fp8(dev(xr))
        wc, ws = o.kv8_encode(xl)
        rwc, rws = o.kv8_encode(xr)
        assert_bytes_equal(host(c), wc, "fp8 codes")
        assert_bytes_equal(host(s), ws, "fp8 scales")
        assert_bytes_equal(host(rc), rwc, "fp8 rope codes")
        assert_bytes_equal(host(rs), rws, "fp8 rope scales")
        return kq.Cache.fp8(c, s, rope=(rc, rs)), o.kv8_decode(wc, ws), o.kv8_decode(rwc, rws)
    p, r = kq.kv_encode_tq4(dev(xl), seed)
    rp, rr = kq.kv_encode_tq4(dev(xr), ROPE_SEED)
    wp, wr = o.tq4_encode(xl, seed)
    rwp, rwr = o.tq4_encode(xr, ROPE_SEED)
    assert_bytes_equal(host(p), wp, "tq4 packed")
    assert_bytes_equal(host(r), wr, "tq4 radius")
    assert_bytes_equal(host(rp), rwp, "tq4 rope packed")
    assert_bytes_equal(host(rr), rwr, "tq4 rope radius")
    return (kq.Cache.tq4(p, r, seed, rope=(rp, rr, ROPE_SEED)), o.tq4_decode(wp, wr, seed),
            o.tq4_decode(rwp, rwr, ROPE_SEED))


@pytest.mark.parametrize("fmt,T,H", [("fp8", 1, 16), ("fp8", 33, 16), ("fp8", 5000, 64),
                                     ("fp8", 32768, 64), ("tq4", 1, 16), ("tq4", 129, 32),
                                     ("tq4", 40000, 16), ("fp8", 5000, 8), ("tq4", 3000, 12)])
def test_rope_decode_matrix_core(fmt, T, H):
    """d = 512 + 64 rope on the matrix-core decode: single rows, ragged tiles
    and chunks, several head groups, a partial head group (8, 12 heads)."""
    xl, xr, q = _inputs(T, H, 512, 64, T + H)
    say(f"{fmt} rope encode T={T}")
    cache, kl, kr = _cache(fmt, xl, xr)
    scale = 1 / np.sqrt(576)
    say(f"attn_decode_quant {fmt} rope T={T} H={H}")
    out, lse = kq.attn_decode_quant(cache, dev(q), scale)
    ro, rl, tw = reference(o.attention_decode_rope, q, kl, kr, scale)
    _check(host(out), host(lse), ro, rl, f"{fmt} rope T={T} H={H}", tw)


@pytest.mark.parametrize("fmt,T,H,d,dr", [("fp8", 300, 4, 64, 16), ("fp8", 1000, 8, 512, 64),
                                          ("tq4", 100, 8, 128, 32), ("tq4", 2049, 4, 512, 64),
                                          ("fp8", 70, 2, 1024, 1024), ("tq4", 17, 3, 64, 2)])
def test_rope_decode_general_path(fmt, T, H, d, dr):
    """Shapes outside the matrix-core kernel (other widths, a rope part as
    wide as the latent) run on the general path; 512 + 64 with 8 heads runs
    on the matrix-core kernel with a partial head group."""
    xl, xr, q = _inputs(T, H, d, dr, 3 * T + d + dr)
    say(f"{fmt} rope encode T={T} d={d} dr={dr}")
    cache, kl, kr = _cache(fmt, xl, xr)
    scale = 1 / np.sqrt(d + dr)
    say(f"attn_decode_quant {fmt} rope general T={T} H={H} d={d} dr={dr}")
    out, lse = kq.attn_decode_quant(cache, dev(q), scale)
    ro, rl, tw = reference(o.attention_decode_rope, q, kl, kr, scale)
    _check(host(out), host(lse), ro, rl, f"{fmt} rope general d={d} dr={dr}", tw)


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
def test_rope_unaligned_query_takes_general_path(fmt):
    T, H = 777, 16
    xl, xr, q = _inputs(T, H, 512, 64, 5)
    cache, kl, kr = _cache(fmt, xl, xr)
    buf = torch.zeros(H * 576 + 1, dtype=torch.float32, device="cuda:0")
    qd = buf[1:].view(H, 576)
    qd.copy_(dev(q))
    say(f"attn_decode_quant {fmt} rope unaligned query")
    out, lse = kq.attn_decode_quant(cache, qd, 0.05)
    ro, rl, tw = reference(o.attention_decode_rope, q, kl, kr, 0.05)
    _check(host(out), host(lse), ro, rl, f"{fmt} rope unaligned q", tw)


@pytest.mark.parametrize("fmt,T,S,H", [("fp8", 300, 40, 16), ("fp8", 20004, 4, 64), ("fp8", 1030, 9, 32),
                                       ("tq4", 200, 7, 16), ("tq4", 64, 64, 16), ("fp8", 50, 5, 4)])
def test_rope_prefill_and_multi_token(fmt, T, S, H):
    """Causal prefill / multi-token decode over the rope key (the latest S
    rows are the new tokens)."""
    d, dr = (512, 64) if H % 16 == 0 else (64, 16)
    g = np.random.default_rng(T + S + H)
    xl = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    xr = (g.standard_normal((T, dr)) * 2.0).astype(np.float32)
    q = g.standard_normal((S, H, d + dr)).astype(np.float32)
    cache, kl, kr = _cache(fmt, xl, xr)
    scale = 1 / np.sqrt(d + dr)
    say(f"attn_prefill_quant {fmt} rope T={T} S={S} H={H}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), T - S, scale)
    ro, rl, tw = reference(o.attention_prefill_rope, q, kl, kr, scale, T - S)
    _check(host(out).reshape(S * H, d), host(lse).reshape(-1), ro, rl, f"{fmt} rope prefill S={S}", tw)


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
def test_rope_dominant_and_absent(fmt):
    """Rope rows far larger than the latent (the rope factor decides the
    softmax), and a zero rope query part (the latent decides alone)."""
    T, H = 3000, 32
    xl, xr, q = _inputs(T, H, 512, 64, 17, rope_gain=200.0)
    q[:, 512:] *= 0.05
    q[3, 512:] = 0.0
    q[4, :512] = 0.0
    cache, kl, kr = _cache(fmt, xl, xr)
    say(f"attn_decode_quant {fmt} rope dominant")
    out, lse = kq.attn_decode_quant(cache, dev(q), 0.04)
    ro, rl, tw = reference(o.attention_decode_rope, q, kl, kr, 0.04)
    _check(host(out), host(lse), ro, rl, f"{fmt} rope dominant", tw)


@pytest.mark.parametrize("fmt,T,k,H", [("fp8", 32768, 2048, 64), ("tq4", 16384, 2048, 16),
                                       ("fp8", 3000, 40, 16)])
def test_rope_gather(fmt, T, k, H):
    """Top-k gather decode over the rope key: listed rows with repeats,
    entries past the cache and -1 padding."""
    xl, xr, q = _inputs(T, H, 512, 64, T + k)
    idx = synth.topk_rows(T, k, seed=k + 3, n_pad=k // 8 + 1, n_dup=k // 16 + 1, n_out=k // 32 + 1)
    cache, kl, kr = _cache(fmt, xl, xr)
    scale = 1 / np.sqrt(576)
    say(f"attn_decode_gather {fmt} rope top-{k} of {T} H={H}")
    out, lse = kq.attn_decode_gather(cache, dev(idx), dev(q), scale)
    ro, rl, tw = reference(o.attention_decode_gather, q, np.concatenate([kl, kr], axis=1), kl, idx, scale)
    _check(host(out), host(lse), ro, rl, f"{fmt} rope gather top-{k}", tw)
