"""Pins for the oracle's float64 attention (decode and causal prefill)."""
import math

import numpy as np

from oracle import kvq_oracle as o


def _bruteforce(q, K, V, scale):
    """Pure-Python loops: softmax(q.k * scale) . V for one head."""
    s = [scale * sum(float(q[i]) * float(K[t][i]) for i in range(len(q))) for t in range(len(K))]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    l = sum(w)
    out = [sum(w[t] * float(V[t][i]) for t in range(len(K))) / l for i in range(len(q))]
    return out, m + math.log(l)


def test_decode_matches_bruteforce_tiny():
    g = np.random.default_rng(0)
    T, H, d = 24, 3, 8
    x = g.standard_normal((T, d))
    q = g.standard_normal((H, d)).astype(np.float32)
    out, lse = o.attention_decode(q, x, x, 0.35)
    for h in range(H):
        ref, rl = _bruteforce(q[h], x, x, 0.35)
        assert np.allclose(out[h], ref, rtol=1e-13, atol=1e-13)
        assert abs(lse[h] - rl) < 1e-12


def test_gqa_grouping_is_contiguous():
    g = np.random.default_rng(1)
    T, n_kv, d, Hq = 16, 2, 8, 8
    K = g.standard_normal((T, n_kv, d))
    V = g.standard_normal((T, n_kv, d))
    q = g.standard_normal((Hq, d))
    out, _ = o.attention_decode(q, K, V, 0.5)
    for h in range(Hq):
        kv = 0 if h < 4 else 1
        ref, _ = _bruteforce(q[h], K[:, kv], V[:, kv], 0.5)
        assert np.allclose(out[h], ref, rtol=1e-13, atol=1e-13)


def test_closed_forms():
    g = np.random.default_rng(2)
    x = g.standard_normal((50, 16))
    q = g.standard_normal((2, 16))
    out, lse = o.attention_decode(q, x[:1], x[:1], 1.0)      # T = 1: the row itself
    assert np.allclose(out, x[0]) and np.allclose(lse, x[:1] @ q.T)
    out, lse = o.attention_decode(np.zeros((2, 16)), x, x, 1.0)   # q = 0: plain mean
    assert np.allclose(out, x.mean(0), rtol=1e-14) and np.allclose(lse, math.log(50))
    rep = np.repeat(x[3:4], 20, axis=0)                      # identical rows: that row
    out, _ = o.attention_decode(q, rep, rep, 0.7)
    assert np.allclose(out, x[3], rtol=1e-14)


def test_lse_is_logsumexp_and_stable():
    g = np.random.default_rng(3)
    x = g.standard_normal((200, 32)) * 30
    q = g.standard_normal((1, 32)) * 30
    out, lse = o.attention_decode(q, x, x, 1.0)
    s = x @ q[0]
    m = s.max()
    assert abs(lse[0] - (m + math.log(np.exp(s - m).sum()))) < 1e-9
    assert np.all(np.isfinite(out))


def test_prefill_is_prefix_decode():
    g = np.random.default_rng(4)
    T, S, H, d = 40, 6, 2, 8
    pos0 = T - S
    x = g.standard_normal((T, d))
    q = g.standard_normal((S, H, d))
    out, lse = o.attention_prefill(q, x, x, 0.4, pos0)
    k = 0
    for s in range(S):
        for h in range(H):
            ref, rl = _bruteforce(q[s, h], x[:pos0 + s + 1], x[:pos0 + s + 1], 0.4)
            assert np.allclose(out[k], ref, rtol=1e-13, atol=1e-13)
            assert abs(lse[k] - rl) < 1e-12
            k += 1


def test_prefill_all_pairs_gqa_matches_bruteforce():
    """The all-pairs prefill (heads of a KV head at once) equals the
    pure-Python brute force per (s, h) with contiguous GQA grouping."""
    g = np.random.default_rng(14)
    T, S, Hq, n_kv, d = 30, 5, 6, 2, 8
    pos0 = T - S
    K = g.standard_normal((T, n_kv, d))
    V = g.standard_normal((T, n_kv, d))
    q = g.standard_normal((S, Hq, d))
    out, lse = o.attention_prefill(q, K, V, 0.3, pos0)
    sub, subl = o.attention_prefill(q, K, V, 0.3, pos0, rows=[(s, h) for s in range(S) for h in range(Hq)])
    assert np.allclose(out, sub, rtol=1e-13, atol=1e-13) and np.allclose(lse, subl, rtol=1e-13)
    k = 0
    for s in range(S):
        for h in range(Hq):
            kv = h // (Hq // n_kv)
            ref, rl = _bruteforce(q[s, h], K[:pos0 + s + 1, kv], V[:pos0 + s + 1, kv], 0.3)
            assert np.allclose(out[k], ref, rtol=1e-13, atol=1e-13)
            assert abs(lse[k] - rl) < 1e-12
            k += 1


def test_rel_l2_definition():
    a = np.array([[3.0, 4.0]])
    assert o.rel_l2(a, a) == 0.0
    assert abs(o.rel_l2(np.array([[3.0, 5.0]]), a) - 0.2) < 1e-15


def test_gather_decode_pins():
    """attention_decode_gather against its definition's closed forms: the
    identity list is the dense decode, a list is the decode over the gathered
    rows computed by pure-Python loops (a repeated row weighted twice),
    padding entries change nothing, and an all-padding list gives 0 / -inf."""
    g = np.random.default_rng(11)
    T, H, d = 40, 3, 8
    x = g.standard_normal((T, d))
    q = g.standard_normal((H, d)).astype(np.float32)
    out, lse = o.attention_decode_gather(q, x, x, np.arange(T), 0.3)
    ro, rl = o.attention_decode(q, x, x, 0.3)
    assert np.array_equal(out, ro) and np.array_equal(lse, rl)
    idx = [7, 3, 3, 39, 0, 12]
    out, lse = o.attention_decode_gather(q, x, x, np.array(idx), 0.3)
    rows = [x[i] for i in idx]
    for h in range(H):
        ref, rlh = _bruteforce(q[h], rows, rows, 0.3)
        assert np.allclose(out[h], ref, rtol=1e-13, atol=1e-13)
        assert abs(lse[h] - rlh) < 1e-12
    # a row listed twice counts twice: weight 2 exp(s) against once
    two, _ = o.attention_decode_gather(q, x, x, np.array([5, 5, 9]), 0.3)
    s5, s9 = 0.3 * (x[5] @ q[0].astype(np.float64)), 0.3 * (x[9] @ q[0].astype(np.float64))
    w5, w9 = 2 * math.exp(s5), math.exp(s9)
    assert np.allclose(two[0], (w5 * x[5] + w9 * x[9]) / (w5 + w9), rtol=1e-13, atol=1e-13)
    padded, plse = o.attention_decode_gather(q, x, x, np.array([-1, 7, T, 3, -5, 3, 39, 0, 12, T + 9]), 0.3)
    assert np.array_equal(padded, out) and np.array_equal(plse, lse)
    z, zl = o.attention_decode_gather(q, x, x, np.array([-1, T, -7]), 0.3)
    assert np.all(z == 0.0) and np.all(np.isneginf(zl))


def test_rope_key_pins():
    """attention_decode_rope / attention_prefill_rope against their
    definition: the general attention over the concatenated key [latent |
    rope] with the latent as value, pure-Python brute force with the two
    partial dots written out, the rope-free case, T = 1, and causal prefill
    rows equal to decodes over the visible prefix."""
    g = np.random.default_rng(21)
    T, H, d, dr = 30, 3, 8, 4
    Kl = g.standard_normal((T, d))
    Kr = g.standard_normal((T, dr)) * 3.0
    q = g.standard_normal((H, d + dr))
    out, lse = o.attention_decode_rope(q, Kl, Kr, 0.4)
    ro, rl = o.attention_decode(q, np.concatenate([Kl, Kr], axis=1), Kl, 0.4)
    assert np.allclose(out, ro, rtol=1e-13, atol=1e-13) and np.allclose(lse, rl, rtol=1e-13)
    assert out.shape == (H, d)
    for h in range(H):
        sc = []
        for t in range(T):
            a = sum(float(q[h, c]) * float(Kl[t, c]) for c in range(d))
            b = sum(float(q[h, d + c]) * float(Kr[t, c]) for c in range(dr))
            sc.append(0.4 * (a + b))
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        L = sum(w)
        for c in range(d):
            assert abs(out[h, c] - sum(w[t] * Kl[t, c] for t in range(T)) / L) < 1e-12
        assert abs(lse[h] - (m + math.log(L))) < 1e-12
    # the rope term moves the weights: dropping it is not a no-op ...
    base, _ = o.attention_decode(q[:, :d], Kl, Kl, 0.4)
    assert not np.allclose(out, base, atol=1e-6)
    # ... and with zero rope rows (or a zero rope query) it is the latent decode
    z, zl = o.attention_decode_rope(q, Kl, np.zeros_like(Kr), 0.4)
    assert np.allclose(z, base, rtol=1e-13, atol=1e-13)
    q0 = q.copy()
    q0[:, d:] = 0.0
    z2, _ = o.attention_decode_rope(q0, Kl, Kr, 0.4)
    assert np.allclose(z2, base, rtol=1e-13, atol=1e-13)
    # one row: the output is that row's latent part, lse its score
    one, ol = o.attention_decode_rope(q, Kl[:1], Kr[:1], 0.4)
    assert np.allclose(one, np.repeat(Kl[:1], H, axis=0), rtol=1e-14)
    assert np.allclose(ol, 0.4 * (q[:, :d] @ Kl[0] + q[:, d:] @ Kr[0]), rtol=1e-13)
    # prefill: query s sees rows t <= pos0 + s
    S, pos0 = 4, T - 4
    qp = g.standard_normal((S, H, d + dr))
    po, pl = o.attention_prefill_rope(qp, Kl, Kr, 0.4, pos0)
    for s in range(S):
        do, dl = o.attention_decode_rope(qp[s], Kl[:pos0 + s + 1], Kr[:pos0 + s + 1], 0.4)
        assert np.allclose(po[s * H:(s + 1) * H], do, rtol=1e-13, atol=1e-13)
        assert np.allclose(pl[s * H:(s + 1) * H], dl, rtol=1e-13)
    sub, _ = o.attention_prefill_rope(qp, Kl, Kr, 0.4, pos0, rows=[(2, 1), (0, 0)])
    assert np.allclose(sub[0], po[2 * H + 1]) and np.allclose(sub[1], po[0])
