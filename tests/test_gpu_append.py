"""GPU q2k appends (kv_append_q2k) vs the oracle's q2k_append, byte for byte,
and attention over appended caches vs the float64 oracle.

Append patterns follow the page's list: decode (one cell per call),
speculative-verify windows of 2-5 cells, 6-step writers, prefill chunks that
start or end mid-group, a prompt of whole groups then decode.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import kvq_oracle as o
from tests._gpu import check_attention, reference, assert_bytes_equal, dev, host, host_u16, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_kv_cache_e4m3_amd as kq

GAIN = 1.10


def _kv(T, n_kv, d, seed, sigma=1.5):
    g = np.random.default_rng(seed)
    gk = np.exp(sigma * g.standard_normal((n_kv, d)))
    gv = np.exp(sigma * g.standard_normal((n_kv, d)))
    K = (g.standard_normal((T, n_kv, d)) * gk).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * gv).astype(np.float32)
    return K, V


def _gpu_appends(K, V, steps, S, W, slack):
    T, n_kv, d = K.shape
    Kd, Vd = dev(K), dev(V)
    buf = kq.q2k_alloc(T, n_kv, d, S, W, slack)
    n = 0
    for st in steps:
        kq.kv_append_q2k(Kd[:n + st], Vd[:n + st], n, GAIN, S, W, slack, buf)
        n += st
    assert n == T
    return buf


def _oracle_appends(K, V, steps, S, W, slack):
    T, n_kv, d = K.shape
    st = o.q2k_empty_state(T, n_kv, d, S, W, slack)
    n = 0
    for step in steps:
        st = o.q2k_append(st, K, V, n, step, GAIN, S, W, slack)
        n += step
    return st


def _same_bytes(buf, st, what):
    assert_bytes_equal(host(buf["k_codes"]), st["k_codes"], what + " k_codes")
    assert_bytes_equal(host_u16(buf["k_scale"]), st["k_scale"], what + " k_scale")
    assert_bytes_equal(host(buf["v_blocks"]), st["v_blocks"], what + " v_blocks")
    if buf["k_ovl"] is not None:
        assert_bytes_equal(host_u16(buf["k_ovl"]), st["k_ovl"], what + " k_ovl")
        assert_bytes_equal(host_u16(buf["v_ovl"]), st["v_ovl"], what + " v_ovl")


def _spec_steps(T, seed):
    g = np.random.default_rng(seed)
    out = []
    while sum(out) < T:
        out.append(int(min(g.integers(2, 6), T - sum(out))))
    return out


@pytest.mark.parametrize("pattern", ["one_call", "decode", "spec", "six", "chunks", "prompt_decode"])
def test_append_bytes_match_oracle(pattern):
    T, n_kv, d, S, W, slack = 203, 2, 256, 8, 40, 16
    K, V = _kv(T, n_kv, d, 31)
    steps = {"one_call": [T], "decode": [1] * T, "spec": _spec_steps(T, 3),
             "six": [6] * (T // 6) + [T % 6], "chunks": [100, 50, 53],
             "prompt_decode": [96] + [1] * (T - 96)}[pattern]
    say(f"kv_append_q2k {pattern} ({len(steps)} calls) T={T}")
    buf = _gpu_appends(K, V, steps, S, W, slack)
    st = _oracle_appends(K, V, steps, S, W, slack)
    _same_bytes(buf, st, pattern)


@pytest.mark.parametrize("n_kv,d,S,W,slack", [(1, 32, 0, 0, 0), (3, 64, 5, 100, 16), (2, 512, 8, 7, 3)])
def test_append_shapes_and_split_invariance(n_kv, d, S, W, slack):
    """Widths, head counts and overlay shapes; every split stores the bytes of
    the one-call append (checked against the oracle too)."""
    T = 130
    K, V = _kv(T, n_kv, d, n_kv * 100 + d)
    say(f"kv_append_q2k shapes n_kv={n_kv} d={d} S={S} W={W} slack={slack}")
    one = _gpu_appends(K, V, [T], S, W, slack)
    _same_bytes(one, _oracle_appends(K, V, [T], S, W, slack), "one call")
    for steps in ([1] * T, [33, 31, 2, 64], _spec_steps(T, 9)):
        buf = _gpu_appends(K, V, steps, S, W, slack)
        for name in ("k_codes", "k_scale", "v_blocks", "k_ovl", "v_ovl"):
            if buf[name] is not None:
                assert torch.equal(buf[name], one[name]), (name, steps[:3])


def test_one_shot_encoder_equals_append():
    """kv_encode_q2k (whole groups) stores what one append call from an empty
    cache stores with no slack."""
    T, n_kv, d, S, W = 256, 2, 256, 8, 64
    K, V = _kv(T, n_kv, d, 41)
    enc = kq.kv_encode_q2k(dev(K), dev(V), GAIN, S, W)
    buf = _gpu_appends(K, V, [T], S, W, 0)
    for name in ("k_codes", "k_scale", "v_blocks", "k_ovl", "v_ovl"):
        assert torch.equal(enc[name], buf[name]), name


@pytest.mark.parametrize("T,steps_kind,Hq", [(203, "decode", 16), (171, "spec", 16),
                                             (4096 + 77, "chunks", 16), (203, "decode", 4),
                                             (32768 + 5, "chunks", 16)])
def test_attention_over_appended_cache(T, steps_kind, Hq):
    """Decode attention over an appended cache, with a partial last group and
    with whole groups only (16 heads: matrix-core path, its last group masked;
    4 heads: general path) vs the oracle over the same bytes."""
    n_kv, d, S, W, slack = 2, 256, 8, 40, 16
    K, V = _kv(T, n_kv, d, T)
    steps = {"decode": [64] + [1] * (T - 64), "spec": _spec_steps(T, 5),
             "chunks": [2048, 1000, 1048] + [2048] * ((T - 4096) // 2048) + [(T - 4096) % 2048]}[steps_kind]
    buf = _gpu_appends(K, V, steps, S, W, slack)
    q = np.random.default_rng(T + 1).standard_normal((Hq, d)).astype(np.float32)
    for n_cells in (T, (T // 32) * 32):          # partial last group, then whole groups only
        cache = kq.Cache.q2k(buf, S, W, slack, n_cells=n_cells)
        say(f"attn_decode_quant q2k appended T={n_cells} ({steps_kind})")
        out, lse = kq.attn_decode_quant(cache, dev(q), 1 / 16)
        kc, ks = host(buf["k_codes"]), host_u16(buf["k_scale"])
        Kd, Vd = o.q2k_decode(kc, ks, host(buf["v_blocks"]), host_u16(buf["k_ovl"]),
                              host_u16(buf["v_ovl"]), S, W, slack, n_cells)
        ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, 1 / 16)
        check_attention(host(out), host(lse), ro, rl, f"appended T={n_cells}", twin=tw)


def test_append_workload_full_size():
    """The q2k decode workload's 32768 cells appended as a 2048-cell prefill
    chunk stream that falls mid-group after a reused 1000-cell prefix, then 37
    decode steps: bytes equal to the oracle's, attention within 1e-5."""
    w = synth.WORKLOADS["q2k_decode"]
    K, V, q = synth.q2k_inputs(w)
    T = w.T
    steps = [1000]
    while sum(steps) + 2048 <= T - 37:
        steps.append(2048)
    steps.append(T - 37 - sum(steps))
    steps += [1] * 37
    say(f"kv_append_q2k full workload ({len(steps)} calls)")
    buf = _gpu_appends(K, V, steps, w.n_sink, w.n_window, 16)
    st = _oracle_appends(K, V, steps, w.n_sink, w.n_window, 16)
    _same_bytes(buf, st, "q2k workload appends")
    cache = kq.Cache.q2k(buf, w.n_sink, w.n_window, 16, n_cells=T)
    out, lse = kq.attn_decode_quant(cache, dev(q), w.sm_scale)
    Kd, Vd = o.q2k_decode(st["k_codes"], st["k_scale"], st["v_blocks"], st["k_ovl"], st["v_ovl"],
                          w.n_sink, w.n_window, 16, T)
    ro, rl, tw = reference(o.attention_decode, q, Kd, Vd, w.sm_scale)
    check_attention(host(out), host(lse), ro, rl, "q2k appended workload", twin=tw)


@pytest.mark.parametrize("T,S,Hq", [(203, 5, 16), (171, 3, 4), (1000, 40, 16)])
def test_q2k_multi_token_over_appended_cache(T, S, Hq):
    """Speculative verify over q2k: the last S cells appended as one window,
    then S query tokens attend causally over the cache (overlay from the ring,
    a partial last group) -- general path -- vs the oracle over the same bytes."""
    n_kv, d, Sk, W, slack = 2, 256, 8, 40, 16
    K, V = _kv(T, n_kv, d, T + S)
    buf = _gpu_appends(K, V, [T - S, S], Sk, W, slack)
    st = _oracle_appends(K, V, [T - S, S], Sk, W, slack)
    _same_bytes(buf, st, f"verify window S={S}")
    q = np.random.default_rng(S).standard_normal((S, Hq, d)).astype(np.float32)
    cache = kq.Cache.q2k(buf, Sk, W, slack, n_cells=T)
    say(f"attn_prefill_quant q2k appended T={T} S={S} Hq={Hq}")
    out, lse = kq.attn_prefill_quant(cache, dev(q), T - S, 1 / 16)
    Kd, Vd = o.q2k_decode(st["k_codes"], st["k_scale"], st["v_blocks"], st["k_ovl"], st["v_ovl"],
                          Sk, W, slack, T)
    ro, rl, tw = reference(o.attention_prefill, q, Kd, Vd, 1 / 16, T - S)
    check_attention(host(out).reshape(S * Hq, d), host(lse).reshape(-1), ro, rl, f"q2k verify S={S}", twin=tw)
