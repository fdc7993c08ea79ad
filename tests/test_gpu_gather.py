"""GPU top-k gather decode (attention over a listed subset of cached rows) vs
the float64 oracle's attention_decode_gather, and vs the library's own dense
decode for an identity list.

The cache is encoded on the GPU and its bytes checked equal to the oracle's
encoding; the oracle decodes those bytes in float64.  Output within 1e-5
relative L2 and lse within 1e-5 relative error, as for the dense decode.
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
D = 512


def _check(out, lse, ref_out, ref_lse, what, twin):
    check_attention(out, lse, ref_out, ref_lse, what, TOL, twin)


def _rows(T, seed):
    g = np.random.default_rng(seed)
    return (g.standard_normal((T, D)) * np.exp(g.standard_normal(D))).astype(np.float32)


def _cache(fmt, x, seed=4242):
    if fmt == "fp8":
        codes, scales = kq.kv_encode_fp8(dev(x))
        wc, ws = o.kv8_encode(x)
        assert_bytes_equal(host(codes), wc, "fp8 codes")
        assert_bytes_equal(host(scales), ws, "fp8 scales")
        return kq.Cache.fp8(codes, scales), o.kv8_decode(wc, ws)
    packed, radius = kq.kv_encode_tq4(dev(x), seed)
    wp, wr = o.tq4_encode(x, seed)
    assert_bytes_equal(host(packed), wp, "tq4 packed")
    assert_bytes_equal(host(radius), wr, "tq4 radius")
    return kq.Cache.tq4(packed, radius, seed), o.tq4_decode(wp, wr, seed)


def _gather(cache, idx, q, scale, what):
    say(f"attn_decode_gather {what} n_idx={idx.size} q={tuple(q.shape)}")
    out, lse = kq.attn_decode_gather(cache, dev(idx), dev(q), scale)
    return host(out), host(lse)


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
@pytest.mark.parametrize("T,H", [(1, 16), (100, 16), (200, 16), (5000, 64), (32768, 16)])
def test_identity_list_equals_dense_decode(fmt, T, H):
    """idx = 0..T-1 attends exactly the dense decode's rows with the same
    chunking: the outputs must agree bit for bit."""
    x = _rows(T, T + H)
    q = np.random.default_rng(T * 3 + H).standard_normal((H, D)).astype(np.float32)
    say(f"{fmt} encode T={T}")
    cache, _ = _cache(fmt, x)
    od, ld = kq.attn_decode_quant(cache, dev(q), 1 / np.sqrt(D))
    og, lg = _gather(cache, np.arange(T, dtype=np.int32), q, 1 / np.sqrt(D), f"{fmt} identity T={T}")
    assert np.array_equal(host(od), og), f"{fmt} T={T}: gather output differs from dense"
    assert np.array_equal(host(ld), lg), f"{fmt} T={T}: gather lse differs from dense"


@pytest.mark.parametrize("fmt,T,k,H", [("fp8", 32768, 2048, 16), ("fp8", 32768, 2048, 128),
                                       ("fp8", 131072, 2048, 64), ("tq4", 16384, 2048, 64),
                                       ("fp8", 4000, 37, 32), ("tq4", 3000, 1, 16),
                                       ("fp8", 50000, 20000, 16), ("fp8", 32768, 2048, 8),
                                       ("tq4", 9000, 700, 3)])
def test_topk_list_matches_oracle(fmt, T, k, H):
    """Random top-k selections with repeats, entries past the cache and -1
    padding; short lists (one chunk, written directly) and long ones (split
    and combined)."""
    x = _rows(T, 7 * T + k)
    q = np.random.default_rng(k + H).standard_normal((H, D)).astype(np.float32)
    idx = synth.topk_rows(T, k, seed=T + k, n_pad=k // 8, n_dup=k // 16, n_out=k // 32)
    say(f"{fmt} encode T={T}")
    cache, xh = _cache(fmt, x)
    out, lse = _gather(cache, idx, q, 1 / np.sqrt(D), f"{fmt} top-{k} of {T} H={H}")
    ro, rl, tw = reference(o.attention_decode_gather, q, xh, xh, idx, 1 / np.sqrt(D))
    _check(out, lse, ro, rl, f"{fmt} top-{k} of {T} H={H}", tw)


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
def test_leading_padding_and_sparse_valid_entries(fmt):
    """Whole tiles and whole chunks of padding before, between and after the
    valid entries (the running maximum starts late; some chunks hold none)."""
    T, H = 6000, 32
    x = _rows(T, 99)
    q = np.random.default_rng(98).standard_normal((H, D)).astype(np.float32)
    g = np.random.default_rng(97)
    idx = np.full(9000, -1, np.int32)
    pos = np.sort(g.choice(9000, 50, replace=False))
    pos[0] = 4000                                       # no valid entry in the first 4000
    pos = np.unique(pos)
    idx[pos] = g.integers(0, T, pos.size)
    idx[8000:8100] = T + 5                              # past the cache: skipped too
    idx[8100:8110] = np.iinfo(np.int32).max             # extreme entries: padding as well
    idx[8110:8120] = np.iinfo(np.int32).min
    say(f"{fmt} encode T={T}")
    cache, xh = _cache(fmt, x)
    out, lse = _gather(cache, idx, q, 1 / np.sqrt(D), f"{fmt} sparse valid entries")
    ro, rl, tw = reference(o.attention_decode_gather, q, xh, xh, idx, 1 / np.sqrt(D))
    _check(out, lse, ro, rl, f"{fmt} sparse valid entries", tw)


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
@pytest.mark.parametrize("n", [5, 3000])
def test_all_padding_list(fmt, n):
    """No valid entry (direct and split plans): out = 0 and lse = -inf, as the
    oracle's reading states."""
    T, H = 500, 16
    x = _rows(T, 5)
    q = np.random.default_rng(6).standard_normal((H, D)).astype(np.float32)
    idx = np.full(n, -1, np.int32)
    idx[::3] = T                                        # one past the last row
    cache, xh = _cache(fmt, x)
    out, lse = _gather(cache, idx, q, 1 / np.sqrt(D), f"{fmt} all padding n={n}")
    ro, rl, tw = reference(o.attention_decode_gather, q, xh, xh, idx, 1 / np.sqrt(D))
    assert np.all(ro == 0.0) and np.all(rl == -np.inf)
    assert np.array_equal(out, np.zeros_like(out)), "expected zeros"
    assert np.all(lse == -np.inf), lse


def test_gather_lse_optional_and_deterministic():
    T, H = 20000, 64
    x = _rows(T, 11)
    q = np.random.default_rng(12).standard_normal((H, D)).astype(np.float32)
    idx = synth.topk_rows(T, 2048, seed=13, n_pad=100, n_dup=20)
    cache, _ = _cache("fp8", x)
    say("gather twice, then without lse")
    o1, l1 = kq.attn_decode_gather(cache, dev(idx), dev(q), 1 / np.sqrt(D))
    o2, l2 = kq.attn_decode_gather(cache, dev(idx), dev(q), 1 / np.sqrt(D))
    o3, l3 = kq.attn_decode_gather(cache, dev(idx), dev(q), 1 / np.sqrt(D), want_lse=False)
    assert l3 is None
    assert np.array_equal(host(o1), host(o2)) and np.array_equal(host(l1), host(l2))
    assert np.array_equal(host(o1), host(o3))
