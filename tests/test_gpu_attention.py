"""GPU attention over encoded caches vs the float64 oracle.

The cache is encoded on the GPU (its bytes are checked equal to the oracle's
own encoding first), the oracle decodes those bytes in float64 and runs
softmax attention; the GPU output must be within 1e-5 relative L2 of it (the
bar the task states for attention), and lse within the same relative error.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import kvq_oracle as o
from tests._gpu import check_attention, reference, DEV, assert_bytes_equal, dev, host, host_u16, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_kv_cache_e4m3_amd as kq

TOL = 1e-5


def _check(out, lse, ref_out, ref_lse, what, twin):
    check_attention(out, lse, ref_out, ref_lse, what, TOL, twin)


def _fp8_cache(x):
    codes, scales = kq.kv_encode_fp8(dev(x))
    wc, ws = o.kv8_encode(x)
    assert_bytes_equal(host(codes), wc, "fp8 codes")
    assert_bytes_equal(host(scales), ws, "fp8 scales")
    return kq.Cache.fp8(codes, scales), o.kv8_decode(wc, ws)


def _tq4_cache(x, seed):
    packed, radius = kq.kv_encode_tq4(dev(x), seed)
    wp, wr = o.tq4_encode(x, seed)
    assert_bytes_equal(host(packed), wp, "tq4 packed")
    assert_bytes_equal(host(radius), wr, "tq4 radius")
    return kq.Cache.tq4(packed, radius, seed), o.tq4_decode(wp, wr, seed)


def _q2k_cache(K, V, gain, ns, nw):
    enc = kq.kv_encode_q2k(dev(K), dev(V), gain, ns, nw)
    kc, ks, vb, ko, vo = o.q2k_encode(K, V, gain, ns, nw)
    assert_bytes_equal(host(enc["k_codes"]), kc, "q2k k_codes")
    assert_bytes_equal(host_u16(enc["k_scale"]), ks, "q2k k_scale")
    assert_bytes_equal(host(enc["v_blocks"]), vb, "q2k v_blocks")
    Kd, Vd = o.q2k_decode(kc, ks, vb, ko if ns + nw else None, vo if ns + nw else None, ns, nw)
    return kq.Cache.q2k(enc, ns, nw), Kd, Vd


def _decode(cache, q, scale, what):
    say(f"attn_decode_quant {what} q={tuple(q.shape)}")
    out, lse = kq.attn_decode_quant(cache, dev(q), scale)
    return host(out), host(lse)


# ---------------------------------------------------------------- KV8 decode

def test_kv8_decode_tiny_workload():
    w = synth.WORKLOADS["tiny_kv8"]
    x, q = synth.latent_inputs(w)
    say("kv8 tiny encode")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, w.sm_scale, "tiny T=256 H=4 d=64")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, w.sm_scale)
    _check(out, lse, ro, rl, "tiny", tw)


def test_kv8_decode_mla_workload_full():
    w = synth.WORKLOADS["kv8_decode"]
    x, q = synth.latent_inputs(w)
    say("kv8 32k encode")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, w.sm_scale, "kv8 T=32768 H=64 d=512")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, w.sm_scale)
    _check(out, lse, ro, rl, "kv8 32k", tw)


def test_kv8_decode_all_heads_workgroup():
    """KV8 decode of 64 heads over a cache long enough (196608 rows and more)
    for one workgroup per chunk to take all four head groups; 200001 rows
    leave a ragged last chunk and tile."""
    T, d, H = 200001, 512, 64
    g = np.random.default_rng(T)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"kv8 encode T={T} d=512")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"kv8 all-heads T={T}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"kv8 all-heads T={T}", tw)


@pytest.mark.parametrize("T,H,d", [(1, 4, 64), (17, 1, 64), (1000, 8, 128), (3001, 64, 512),
                                   (777, 16, 1024), (50, 3, 40)])
def test_kv8_decode_ragged(T, H, d):
    g = np.random.default_rng(T + H + d)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"kv8 encode T={T} d={d}")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"kv8 T={T} H={H} d={d}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"kv8 T={T}", tw)


@pytest.mark.parametrize("T,H", [(1, 16), (33, 16), (128, 32), (129, 64), (5000, 128), (32768, 16),
                                 (40000, 48)])
def test_kv8_decode_matrix_core_shapes(T, H):
    """d = 512 with heads in groups of 16 runs on the MFMA decode path:
    single rows, ragged tiles and chunks, several head-group counts."""
    d = 512
    g = np.random.default_rng(T * 11 + H)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"kv8 encode T={T} d=512")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"kv8 mfma T={T} H={H}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"kv8 mfma T={T} H={H}", tw)


@pytest.mark.parametrize("T,H", [(32768, 8), (1000, 1), (5000, 24), (129, 40), (3001, 5)])
def test_kv8_decode_partial_head_group(T, H):
    """d = 512 with a head count that is not a multiple of 16: the last head
    group of the matrix-core decode holds fewer heads (zero queries in the
    rest, nothing written for them)."""
    d = 512
    g = np.random.default_rng(T * 13 + H)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"kv8 encode T={T} d=512")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"kv8 mfma partial group T={T} H={H}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"kv8 mfma partial group T={T} H={H}", tw)


@pytest.mark.parametrize("T,S,H", [(2000, 3, 8), (700, 2, 20)])
def test_kv8_multi_token_partial_head_group(T, S, H):
    d = 512
    x, q = _prefill_small(T, S, H, d, T + 5 * S + H)
    pos0 = T - S
    cache, xh = _fp8_cache(x)
    say(f"attn_prefill_quant partial head group T={T} S={S} H={H}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), pos0, 1 / np.sqrt(d))
    ro, rl, tw = reference(o.attention_prefill, q, xh, xh, 1 / np.sqrt(d), pos0)
    _check(host(out).reshape(S * H, d), host(lse).reshape(-1), ro, rl, f"multi-token H={H} S={S}", tw)


def test_kv8_decode_scaled_queries_and_rows():
    """Query and row magnitudes far from 1 (the f16 split pre-scales both)."""
    d, T, H = 512, 2000, 32
    g = np.random.default_rng(5)
    x = (g.standard_normal((T, d)) * 1e-3).astype(np.float32)
    x[::7] *= 1e5                                       # rows with very different scales
    q = (g.standard_normal((H, d)) * 3e3).astype(np.float32)
    q[1] *= 1e-6                                        # a nearly-zero query head
    q[2] = 0.0                                          # an exactly zero query head
    say("kv8 encode scaled rows")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), "kv8 mfma scaled")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, "kv8 mfma scaled", tw)


def test_kv8_decode_edge_rows_and_peaked_softmax():
    d = 64
    x = np.concatenate([synth.edge_rows(d)[:-3], np.random.default_rng(0).standard_normal((40, d))]).astype(np.float32)
    q = (np.random.default_rng(1).standard_normal((4, d)) * 30).astype(np.float32)   # very peaked
    say("kv8 edge encode")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 0.125, "kv8 edge rows, peaked")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 0.125)
    _check(out, lse, ro, rl, "edge", tw)


# ---------------------------------------------------------------- TQ4 decode

# sigma 0: plain N(0,1) rows without channel gains, the other reading of the
# row distribution of the 128k TQ4 decode and the 16k prefill workloads
@pytest.mark.parametrize("sigma", [1.0, 0.0])
def test_tq4_decode_mla_workload_full(sigma):
    w = dataclasses.replace(synth.WORKLOADS["tq4_decode"], sigma=sigma)
    x, q = synth.latent_inputs(w)
    say(f"tq4 128k encode sigma={sigma}")
    packed, radius = kq.kv_encode_tq4(dev(x), synth.ROT_SEED)
    wp, wr = o.tq4_encode(x[:2048], synth.ROT_SEED)              # sampled byte check
    assert_bytes_equal(host(packed)[:2048], wp, "tq4 packed (first 2048 rows)")
    cache = kq.Cache.tq4(packed, radius, synth.ROT_SEED)
    out, lse = _decode(cache, q, w.sm_scale, "tq4 T=131072 H=64 d=512")
    xh = o.tq4_decode(host(packed), host(radius), synth.ROT_SEED)  # oracle decodes the GPU bytes
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, w.sm_scale)
    _check(out, lse, ro, rl, "tq4 128k", tw)


@pytest.mark.parametrize("T,H,d", [(1, 2, 64), (300, 4, 64), (2049, 64, 512), (100, 8, 1024), (40, 2, 8)])
def test_tq4_decode_ragged(T, H, d):
    g = np.random.default_rng(T * 3 + d)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"tq4 encode T={T} d={d}")
    cache, xh = _tq4_cache(x, 12345)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"tq4 T={T} H={H} d={d}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"tq4 T={T}", tw)


@pytest.mark.parametrize("T,H", [(1, 16), (33, 16), (129, 64), (5000, 32), (40000, 48)])
def test_tq4_decode_matrix_core_shapes(T, H):
    """d = 512 TQ4 rows on the MFMA decode path (rotated query, byte-table
    operands, rotated-domain context unrotated in the combine)."""
    d = 512
    g = np.random.default_rng(T * 7 + H)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"tq4 encode T={T} d=512")
    cache, xh = _tq4_cache(x, 0x9E3779B97F4A7C15 ^ T)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"tq4 mfma T={T} H={H}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"tq4 mfma T={T} H={H}", tw)


@pytest.mark.parametrize("T,H", [(40000, 8), (300, 5)])
def test_tq4_decode_partial_head_group(T, H):
    d = 512
    g = np.random.default_rng(T * 5 + H)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"tq4 encode T={T} d=512")
    cache, xh = _tq4_cache(x, 0x51ED27 + T)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"tq4 mfma partial group T={T} H={H}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"tq4 mfma partial group T={T} H={H}", tw)


@pytest.mark.parametrize("T,case", [(77824, "plain"), (80001, "plain"), (90000, "scaled"), (100000, "late_max")])
def test_tq4_decode_all_heads_workgroup(T, case):
    """TQ4 decode of 64 heads over a long cache: one workgroup per chunk takes
    all four head groups and decodes each row once.  77824 rows is the
    smallest cache on that path (304-row chunks, rounded to 320: 10 tiles);
    80001 leaves a ragged last chunk and tile; "scaled" spans radii over three
    decades with zero rows, a zero query head and a nearly-zero one;
    "late_max" puts a row with large scores in the last tile of every chunk,
    so running maxima rise late and the accumulators are rescaled after the
    first tiles."""
    d, H = 512, 64
    g = np.random.default_rng(T + 17)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    if case == "scaled":
        # (radii over three decades: with the 1e-2 / 1e2 spread of the shorter
        # test the largest scores here reach several hundred, where float32
        # scores alone move a row by more than the bar)
        x *= 1e-1
        x[::5] *= 1e2
        x[3::11] = 0.0
        q[0] = 0.0
        q[1] *= 1e-7
    elif case == "late_max":
        # in the last tile of every chunk (the plan's 256 chunks of ceil(T / 256)
        # rows rounded up to 32), a row aligned with the query of one head
        chunk = ((T + 255) // 256 + 31) // 32 * 32
        for c, c0 in enumerate(range(0, T, chunk)):
            t = min(c0 + chunk - 16, T - 1)
            x[t] = 6.0 * q[c % H] / np.linalg.norm(q[c % H]) * np.sqrt(d)
    say(f"tq4 encode T={T} d=512 {case}")
    cache, xh = _tq4_cache(x, 0xC0FFEE + T)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"tq4 all-heads T={T} {case}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"tq4 all-heads T={T} {case}", tw)


def test_tq4_decode_scaled_and_degenerate_rows():
    """Radii spanning many decades, all-zero rows (radius 0), a zero query head
    and a nearly-zero one."""
    d, T, H = 512, 3000, 32
    g = np.random.default_rng(9)
    x = (g.standard_normal((T, d)) * 1e-2).astype(np.float32)
    x[::5] *= 1e4
    x[3::11] = 0.0
    q = (g.standard_normal((H, d)) * 5.0).astype(np.float32)
    q[0] = 0.0
    q[1] *= 1e-7
    say("tq4 encode scaled rows")
    cache, xh = _tq4_cache(x, 77)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), "tq4 mfma scaled")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, "tq4 mfma scaled", tw)


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
def test_unaligned_query_takes_general_path(fmt):
    """A query that is only 4-byte aligned cannot use 16-byte vector loads; the
    general path must give the same answer to the oracle's tolerance."""
    d, T, H = 512, 700, 16
    g = np.random.default_rng(21)
    x = g.standard_normal((T, d)).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"{fmt} encode for unaligned query")
    cache, xh = _fp8_cache(x) if fmt == "fp8" else _tq4_cache(x, 5)
    buf = torch.empty(H * d + 1, dtype=torch.float32, device=DEV)
    qv = buf[1:].view(H, d)
    qv.copy_(dev(q))
    assert qv.data_ptr() % 16 != 0
    say(f"attn_decode_quant {fmt} unaligned query")
    out, lse = kq.attn_decode_quant(cache, qv, 1 / np.sqrt(d))
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(host(out), host(lse), ro, rl, f"{fmt} unaligned query", tw)


# ---------------------------------------------------------------- q2k decode

def test_q2k_decode_workload_full():
    w = synth.WORKLOADS["q2k_decode"]
    K, V, q = synth.q2k_inputs(w)
    say("q2k 32k encode")
    cache, Kd, Vd = _q2k_cache(K, V, w.k_gain, w.n_sink, w.n_window)
    out, lse = _decode(cache, q, w.sm_scale, "q2k T=32768 16q/2kv d=256")
    ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, w.sm_scale)
    _check(out, lse, ro, rl, "q2k 32k", tw)


@pytest.mark.parametrize("T,n_kv,Hq,d,ns,nw", [(32, 1, 1, 32, 0, 0), (64, 2, 16, 64, 8, 16),
                                              (96, 2, 4, 256, 8, 256), (320, 4, 32, 128, 0, 64),
                                              (1024, 2, 16, 256, 8, 256)])
def test_q2k_decode_shapes(T, n_kv, Hq, d, ns, nw):
    g = np.random.default_rng(T + d + Hq)
    K = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    q = g.standard_normal((Hq, d)).astype(np.float32)
    say(f"q2k encode T={T} n_kv={n_kv} d={d}")
    cache, Kd, Vd = _q2k_cache(K, V, 1.10, ns, nw)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"q2k T={T} n_kv={n_kv} Hq={Hq} d={d}")
    ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"q2k T={T}", tw)


@pytest.mark.parametrize("T,n_kv,ns,nw", [(32, 1, 0, 0), (4096, 2, 8, 256), (2048, 3, 5, 100),
                                         (128, 1, 200, 0), (256, 2, 0, 300), (8192, 1, 40, 31),
                                         (33792, 2, 8, 256)])
def test_q2k_decode_matrix_core_shapes(T, n_kv, ns, nw):
    """d = 256 with 8 query heads per KV head runs on the MFMA q2k path:
    single groups and chunks, overlays that cover part of a group, all of the
    cache or none of it, several KV heads."""
    d, Hq = 256, 8 * n_kv
    g = np.random.default_rng(T * 5 + n_kv * 7 + ns)
    K = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    q = g.standard_normal((Hq, d)).astype(np.float32)
    say(f"q2k encode T={T} n_kv={n_kv} ns={ns} nw={nw}")
    cache, Kd, Vd = _q2k_cache(K, V, 1.10, ns, nw)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"q2k mfma T={T} n_kv={n_kv}")
    ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"q2k mfma T={T} n_kv={n_kv} ns={ns} nw={nw}", tw)


def test_q2k_decode_scaled_and_degenerate():
    """Magnitudes far from 1 in K, V and the query, all-zero cells and a zero
    query head, with an overlay; a large gain on the stored K scales."""
    d, n_kv, T = 256, 2, 1024
    g = np.random.default_rng(99)
    K = (g.standard_normal((T, n_kv, d)) * 1e-3).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * 3e2).astype(np.float32)
    K[::9] *= 1e4
    V[5::13] *= 1e-5
    K[64:96] = 0.0
    V[96:128] = 0.0
    q = (g.standard_normal((16, d)) * 40.0).astype(np.float32)
    q[3] = 0.0
    say("q2k encode scaled")
    cache, Kd, Vd = _q2k_cache(K, V, 2.5, 8, 64)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), "q2k mfma scaled")
    ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, "q2k mfma scaled", tw)


def test_q2k_decode_overlay_outliers():
    """Sink and window cells far larger than the bulk (the outliers the overlay
    exists for): V overlay values ~1e3x the bulk V range and K overlay values
    ~1e4x, so no pre-scale chosen from the bulk alone can hold them in f16."""
    d, n_kv, T = 256, 2, 2048
    g = np.random.default_rng(123)
    K = g.standard_normal((T, n_kv, d)).astype(np.float32)
    V = g.standard_normal((T, n_kv, d)).astype(np.float32)
    K[0:8] *= 1e4
    V[0:8] *= 2e3
    V[T - 5] *= 3e3
    K[T - 40] *= 5e3
    q = (g.standard_normal((16, d)) * 1e-4).astype(np.float32)     # sink scores O(1)
    say("q2k encode overlay outliers")
    cache, Kd, Vd = _q2k_cache(K, V, 1.1, 8, 96)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), "q2k mfma overlay outliers")
    ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, 1 / np.sqrt(d))
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    _check(out, lse, ro, rl, "q2k mfma overlay outliers", tw)


# ---------------------------------------------------------------- KV8 prefill

def _prefill_small(T, S, H, d, seed):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((S, H, d)).astype(np.float32)
    return x, q


@pytest.mark.parametrize("T,S,H,d", [(300, 40, 4, 64), (64, 64, 2, 64), (1030, 7, 64, 512), (5, 1, 3, 16),
                                     # one chunk per token (shared flash-attention tiles):
                                     # S not a multiple of 4, pos0 = 0, 16 heads
                                     (300, 66, 64, 512), (64, 64, 64, 512), (1000, 257, 16, 512),
                                     # the same kernel split over T: 32 chunks of 20 tiles (the last
                                     # 5), and 65 chunks of 2 tiles whose last chunk holds 4 rows
                                     (20000, 8, 64, 512), (4100, 9, 16, 512)])
def test_kv8_prefill_small(T, S, H, d):
    x, q = _prefill_small(T, S, H, d, T + S)
    pos0 = T - S
    say(f"kv8 prefill encode T={T}")
    cache, xh = _fp8_cache(x)
    say(f"attn_prefill_quant T={T} S={S} H={H} d={d}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), pos0, 1 / np.sqrt(d))
    ro, rl, tw = reference(o.attention_prefill, q, xh, xh, 1 / np.sqrt(d), pos0)
    _check(host(out).reshape(S * H, d), host(lse).reshape(-1), ro, rl, f"prefill T={T} S={S}", tw)


@pytest.mark.parametrize("T,S,H,d", [(1030, 7, 64, 512), (300, 40, 4, 64), (200, 130, 16, 512),
                                     (600, 300, 16, 512)])
def test_tq4_prefill_small(T, S, H, d):
    x, q = _prefill_small(T, S, H, d, 3 * T + S)
    pos0 = T - S
    say(f"tq4 prefill encode T={T}")
    cache, xh = _tq4_cache(x, 31337)
    say(f"attn_prefill_quant tq4 T={T} S={S} H={H} d={d}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), pos0, 1 / np.sqrt(d))
    ro, rl, tw = reference(o.attention_prefill, q, xh, xh, 1 / np.sqrt(d), pos0)
    _check(host(out).reshape(S * H, d), host(lse).reshape(-1), ro, rl, f"tq4 prefill T={T} S={S}", tw)


@pytest.mark.parametrize("S", [2, 3, 4, 8, 13])
def test_kv8_multi_token_decode(S):
    """Multi-token decode (verify S new tokens, causal among them) over a long
    cache, split into chunks and merged by the combine."""
    w = synth.WORKLOADS["kv8_decode"]
    T = 20000 + S
    x, _ = synth.latent_inputs(w, T=T)
    q = np.random.default_rng(900 + S).standard_normal((S, w.Hq, w.d)).astype(np.float32)
    say(f"multi-token decode S={S}: encode T={T}")
    cache, xh = _fp8_cache(x)
    say(f"attn_prefill_quant S={S} T={T} H={w.Hq}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), T - S, w.sm_scale)
    ro, rl, tw = reference(o.attention_prefill, q, xh, xh, w.sm_scale, T - S)
    _check(host(out).reshape(S * w.Hq, w.d), host(lse).reshape(-1), ro, rl, f"multi-token S={S}", tw)


@pytest.mark.parametrize("sigma", [1.0, 0.0])
def test_kv8_prefill_workload_full_size(sigma):
    """S=512 new rows over T=16384 (pos0=15872): the new rows are encoded on the
    GPU into the cache first, then every (s, h) pair -- all 32768 -- is
    compared with the oracle.  sigma 0 is the plain N(0,1) reading of the rows."""
    w = dataclasses.replace(synth.WORKLOADS["kv8_prefill"], sigma=sigma)
    x, q = synth.latent_inputs(w)
    say(f"kv8 prefill 16k sigma={sigma}: encode old rows, then the 512 new rows into the cache")
    codes = torch.empty((w.T, w.d), dtype=torch.uint8, device=DEV)
    scales = torch.empty((w.T,), dtype=torch.float32, device=DEV)
    xd = dev(x)
    kq.kv_encode_fp8(xd[:w.pos0], codes[:w.pos0], scales[:w.pos0])
    kq.kv_encode_fp8(xd[w.pos0:], codes[w.pos0:], scales[w.pos0:])
    wc, ws = o.kv8_encode(x)
    assert_bytes_equal(host(codes), wc, "prefill cache codes")
    assert_bytes_equal(host(scales), ws, "prefill cache scales")
    cache = kq.Cache.fp8(codes, scales)
    say("attn_prefill_quant S=512 H=64 d=512 T=16384")
    out, lse = kq.attn_prefill_quant(cache, dev(q), w.pos0, w.sm_scale)
    out, lse = host(out), host(lse)
    xh = o.kv8_decode(wc, ws)
    ro, rl, tw = reference(o.attention_prefill, q, xh, xh, w.sm_scale, w.pos0)
    _check(out.reshape(w.S * w.Hq, w.d), lse.reshape(-1), ro, rl, f"prefill 16k all pairs sigma={sigma}", tw)


def test_decode_is_deterministic():
    w = synth.WORKLOADS["kv8_decode"]
    x, q = synth.latent_inputs(w, T=4096)
    say("determinism: kv8 encode 4096")
    codes, scales = kq.kv_encode_fp8(dev(x))
    cache = kq.Cache.fp8(codes, scales)
    qd = dev(q)
    say("determinism: two decodes")
    a, la = kq.attn_decode_quant(cache, qd, w.sm_scale)
    b, lb = kq.attn_decode_quant(cache, qd, w.sm_scale)
    assert np.array_equal(host(a), host(b)) and np.array_equal(host(la), host(lb))


def test_kv8_prefill_shared_tiles_scaled_rows():
    """The shared-tile prefill (one chunk per token) with row and query
    magnitudes far from 1, zero rows and a zero query head: the weight
    pre-scale comes from the largest row scale a token group sees."""
    d, T, S, H = 512, 700, 70, 64
    g = np.random.default_rng(17)
    x = (g.standard_normal((T, d)) * 1e-3).astype(np.float32)
    x[::11] *= 1e5
    x[40:72] = 0.0
    # scores of the large rows O(1): a 2^-22 relative score error then stays far
    # below the bar (scores of 1e3 would amplify it past 1e-5 in any f32 path)
    q = (g.standard_normal((S, H, d)) * 1e-2).astype(np.float32)
    q[3, 5] = 0.0
    q[9] *= 1e-5
    pos0 = T - S
    say("kv8 prefill scaled: encode")
    cache, xh = _fp8_cache(x)
    say(f"attn_prefill_quant scaled T={T} S={S} H={H}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), pos0, 1 / np.sqrt(d))
    ro, rl, tw = reference(o.attention_prefill, q, xh, xh, 1 / np.sqrt(d), pos0)
    _check(host(out).reshape(S * H, d), host(lse).reshape(-1), ro, rl, "prefill shared tiles scaled", tw)


def test_prefill_is_deterministic_and_lse_optional():
    """Two prefills give identical bits; without lse the output is unchanged."""
    d, T, S, H = 512, 400, 68, 64
    x, q = _prefill_small(T, S, H, d, 4242)
    say("prefill determinism: encode")
    cache, xh = _fp8_cache(x)
    qd = dev(q)
    say("prefill determinism: three prefills")
    a, la = kq.attn_prefill_quant(cache, qd, T - S, 1 / np.sqrt(d))
    b, lb = kq.attn_prefill_quant(cache, qd, T - S, 1 / np.sqrt(d))
    c, lc = kq.attn_prefill_quant(cache, qd, T - S, 1 / np.sqrt(d), want_lse=False)
    assert lc is None
    assert np.array_equal(host(a), host(b)) and np.array_equal(host(la), host(lb))
    assert np.array_equal(host(a), host(c))


@pytest.mark.parametrize("fmt", ["fp8", "tq4"])
def test_decode_long_chunks(fmt):
    """256 heads over T = 40000 rows: 16 head groups leave 16 chunks of 2560 rows
    each, longer than the 2048 rows whose factors the kernel loads up front for
    the weight pre-scale, so the rest of each chunk goes through the follow-up
    pass; the largest row factor of every chunk sits in that rest."""
    T, H, d = 40000, 256, 512
    g = np.random.default_rng(2560)
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    # the largest row factor of each chunk at its row 2500
    x[2500:T:2560] *= 64.0
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"{fmt} encode T={T} for H={H}")
    if fmt == "fp8":
        cache, xh = _fp8_cache(x)
    else:
        cache, xh = _tq4_cache(x, synth.ROT_SEED)
    out, lse = _decode(cache, q, 1 / np.sqrt(d), f"{fmt} T={T} H={H}")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    _check(out, lse, ro, rl, f"{fmt} long chunks", tw)


def test_maximum_head_counts():
    """The largest head counts the calls accept: 4096 query heads over one
    latent (general path, 16 heads per workgroup) and 64 q2k KV heads of 8
    query heads each (matrix-core path)."""
    g = np.random.default_rng(4096)
    x = g.standard_normal((64, 64)).astype(np.float32)
    q = g.standard_normal((4096, 64)).astype(np.float32)
    say("kv8 encode for 4096 heads")
    cache, xh = _fp8_cache(x)
    out, lse = _decode(cache, q, 0.125, "kv8 H=4096 d=64 T=64")
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 0.125)
    _check(out, lse, ro, rl, "kv8 H=4096", tw)
    T, n_kv, d = 64, 64, 256
    K = (g.standard_normal((T, n_kv, d)) * np.exp(g.standard_normal((n_kv, d)))).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * np.exp(g.standard_normal((n_kv, d)))).astype(np.float32)
    qq = g.standard_normal((8 * n_kv, d)).astype(np.float32)
    say("q2k encode n_kv=64")
    qc, Kd, Vd = _q2k_cache(K, V, 1.10, 4, 8)
    out, lse = _decode(qc, qq, 1 / 16, "q2k n_kv=64 Hq=512")
    ro, rl, tw = reference(o.attention_decode, qq, Kd, Vd, 1 / 16)
    _check(out, lse, ro, rl, "q2k n_kv=64", tw)


@pytest.mark.parametrize("T,S,ns,nw", [(4096, 2, 8, 256), (4096, 4, 8, 256), (2048, 37, 5, 100),
                                       (32768, 4, 8, 256), (64, 64, 0, 0)])
def test_q2k_multi_token(T, S, ns, nw):
    """q2k causal attention for S new tokens at the end of the cache
    (speculative verify / chunked prefill) on the matrix-core path: each
    token's causal limit falls inside a 32-cell group."""
    n_kv, d, Hq = 2, 256, 16
    g = np.random.default_rng(T + S)
    K = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    q = g.standard_normal((S, Hq, d)).astype(np.float32)
    say(f"q2k encode T={T}")
    cache, Kd, Vd = _q2k_cache(K, V, 1.10, ns, nw)
    say(f"attn_prefill_quant q2k T={T} S={S}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), T - S, 1 / 16)
    ro, rl, tw = reference(o.attention_prefill, q, Kd, Vd, 1 / 16, T - S)
    _check(host(out).reshape(S * Hq, d), host(lse).reshape(-1), ro, rl, f"q2k S={S} T={T}", tw)
