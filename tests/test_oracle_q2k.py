"""Pins for the oracle's q2k cache (2-bit per-channel K, q4_0 V, fp16 overlay)."""
import struct

import numpy as np
import pytest

from oracle import kvq_oracle as o
from tests._golden import lines, page_numbers


def _kv(T=64, n_kv=2, d=64, seed=0, sigma=1.5):
    g = np.random.default_rng(seed)
    gk = np.exp(sigma * g.standard_normal((n_kv, d)))
    gv = np.exp(sigma * g.standard_normal((n_kv, d)))
    K = (g.standard_normal((T, n_kv, d)) * gk).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * gv).astype(np.float32)
    return K, V


def test_k_gain_changes_only_the_stored_scale():
    # Strata #2318 "Summary" item 3 / "Measurements" (kv_q2_parity K-gain pin):
    # stored scale = B x the rule, codes chosen against the un-gained scale.
    K, _ = _kv()
    c1, s1 = o.q2k_encode_k(K, 1.0)
    c2, s2 = o.q2k_encode_k(K, 1.10)
    c3, s3 = o.q2k_encode_k(K, 2.0)
    assert np.array_equal(c1, c2) and np.array_equal(c1, c3)
    # B = 2 is exact: the half-precision exponent moves up by one
    normal = (s1 & 0x7C00) != 0
    assert np.array_equal(s3[normal], s1[normal] + 0x400)
    r = o.f16_value(s2) / o.f16_value(s1)
    assert np.all(np.abs(r - 1.10) < 2e-3)


def test_k_scale_is_group_rms():
    K, _ = _kv(T=96)
    _, s = o.q2k_encode_k(K, 1.0)
    G = 3
    rms = np.sqrt(np.mean(K.astype(np.float64).reshape(G, 32, 2, 64) ** 2, axis=1))
    assert np.allclose(o.f16_value(s), rms, rtol=2 ** -10)


def test_k_codes_are_nearest_levels():
    K, _ = _kv(T=128, seed=3)
    codes, s = o.q2k_encode_k(K, 1.0)
    G, n_kv, d = 4, 2, 64
    rms = np.sqrt(np.mean(K.astype(np.float64).reshape(G, 32, n_kv, d) ** 2, axis=1))
    lv = o.codebook_f16(4).astype(np.float64)
    b = codes.astype(np.int64)
    cc = np.stack([(b >> (2 * i)) & 3 for i in range(4)], -1).reshape(G, n_kv, d, 32)
    z = K.reshape(G, 32, n_kv, d).transpose(0, 2, 3, 1) / rms[..., None]
    dist = np.abs(z[..., None] - lv)
    best = np.argmin(dist, -1)
    srt = np.sort(dist, -1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-5
    assert np.array_equal(cc[clear], best[clear])


def test_q4_0_decode_rule_golden_block():
    rows = list(lines("q4_0_block_example.txt"))
    blk = np.array([int(t, 16) for t in rows[0].split()[1:]], np.uint8)
    want = np.array([float(t) for t in rows[1].split()[1:]])
    # one cell, one head, d = 32 -> exactly one block
    vb = blk.reshape(1, 1, 1, 18).repeat(32, axis=0)
    _, V = o.q2k_decode(np.zeros((1, 1, 32, 8), np.uint8), np.zeros((1, 1, 32), np.uint16),
                        vb, None, None, 0, 0)
    assert np.array_equal(V[0, 0], want)


def test_q4_0_encode_error_bound_and_extremes():
    _, V = _kv(T=64, seed=5)
    vb = o.q2k_encode_v(V)
    Kd, Vd = o.q2k_decode(np.zeros((2, 2, 64, 8), np.uint8), np.zeros((2, 2, 64), np.uint16),
                          vb, None, None, 0, 0)
    blocks = V.astype(np.float64).reshape(64, 2, 2, 32)
    dec = Vd.reshape(64, 2, 2, 32)
    dv = o.f16_value((vb[..., 0].astype(np.uint16) | (vb[..., 1].astype(np.uint16) << 8)))
    err = np.abs(dec - blocks)
    # half a step, plus the slack from rounding d to half precision (|x|/d <= 7 * (1 + 2^-11))
    assert np.all(err <= dv[..., None] * (0.5 + 7 * 2 ** -10))
    # the amax element decodes to +-7 d
    j = np.argmax(np.abs(blocks), -1)
    top = np.take_along_axis(dec, j[..., None], -1)[..., 0]
    assert np.allclose(np.abs(top), 7 * dv)


def test_zero_blocks_and_groups():
    K = np.zeros((32, 1, 32), np.float32)
    kc, ks, vb, ko, vo = o.q2k_encode(K, K, 1.1, 2, 4)
    assert np.all(kc == 0) and np.all(ks == 0)
    assert np.all(vb[..., :2] == 0) and np.all(vb[..., 2:] == 0x88)
    Kd, Vd = o.q2k_decode(kc, ks, vb, ko, vo, 2, 4)
    assert np.all(Kd == 0) and np.all(Vd == 0)


def test_overlay_slots_and_exact_reads():
    # Strata #2318 "Measurements" (kv_window_parity): sink and window cells read
    # bit-exactly the fp16 values; cells outside read the bulk bit-for-bit.
    T, S, N = 96, 8, 40
    cells = o.overlay_slot_cells(T, S, N)
    live = cells[cells >= 0]
    assert len(set(live.tolist())) == len(live)
    assert set(live.tolist()) == set(range(S)) | set(range(T - N, T))
    K, V = _kv(T=T, seed=9)
    kc, ks, vb, ko, vo = o.q2k_encode(K, V, 1.1, S, N)
    Kd, Vd = o.q2k_decode(kc, ks, vb, ko, vo, S, N)
    Kb, Vb = o.q2k_decode(kc, ks, vb, None, None, S, N)
    for t in range(T):
        if t < S or t >= T - N:
            assert np.array_equal(Kd[t], K[t].astype(np.float16).astype(np.float64))
            assert np.array_equal(Vd[t], V[t].astype(np.float16).astype(np.float64))
        else:
            assert np.array_equal(Kd[t], Kb[t]) and np.array_equal(Vd[t], Vb[t])
    # overlapping sinks and window (T < S + N): no slot collision, unused slots zero
    cells = o.overlay_slot_cells(32, 8, 30)
    live = cells[cells >= 0]
    assert len(set(live.tolist())) == len(live) == 32
    K2, V2 = _kv(T=32, seed=10)
    _, _, _, ko2, _ = o.q2k_encode(K2, V2, 1.1, 8, 30)
    assert np.all(ko2[cells < 0] == 0)


def test_full_overlay_equals_fp16_cache_attention():
    T = 64
    K, V = _kv(T=T, n_kv=2, d=32, seed=11)
    kc, ks, vb, ko, vo = o.q2k_encode(K, V, 1.1, 32, 32)
    Kd, Vd = o.q2k_decode(kc, ks, vb, ko, vo, 32, 32)
    q = np.random.default_rng(1).standard_normal((4, 32)).astype(np.float32)
    a, _ = o.attention_decode(q, Kd, Vd, 0.2)
    b, _ = o.attention_decode(q, K.astype(np.float16).astype(np.float64),
                              V.astype(np.float16).astype(np.float64), 0.2)
    assert np.array_equal(a, b)


def test_q2k_byte_accounting_matches_page():
    p = page_numbers()
    assert o.row_bytes("q2k", 256, 2) == p["q2k_bytes_per_cell"]
    assert o.row_bytes("q2k", 256, 1) == p["q2k_bytes_per_cell_head"]
    gib = 262144 * 12 * o.row_bytes("q2k", 256, 2) / 2 ** 30
    assert abs(gib - p["q2k_total_gib"]) < 0.005
    # the page's other formats from the same rule set: q4_0 K+V, FP16
    q4 = 2 * 2 * (256 // 32) * 18
    assert q4 == p["q4_0_bytes_per_cell"]
    assert abs(262144 * 12 * q4 / 2 ** 30 - p["q4_0_total_gib"]) < 0.005
    assert 2 * 2 * 256 * 2 == p["fp16_bytes_per_cell"]
    # the encoder's arrays add up to that many bytes
    K, V = _kv(T=64, n_kv=2, d=256, seed=2)
    kc, ks, vb, _, _ = o.q2k_encode(K, V, 1.1, 8, 16)
    assert (kc.nbytes + ks.nbytes + vb.nbytes) / 64 == p["q2k_bytes_per_cell"]


# ---------------------------------------------------------------- appends

def _run_appends(K, V, steps, gain=1.1, S=8, W=40, slack=16):
    """Append cells in calls of the given sizes; returns the final state."""
    T, n_kv, d = K.shape
    st = o.q2k_empty_state(T, n_kv, d, S, W, slack)
    n = 0
    for step in steps:
        st = o.q2k_append(st, K, V, n, step, gain, S, W, slack)
        n += step
    assert n == T
    return st


def test_ring_slots_are_fixed_distinct_and_in_range():
    """Strata #2318 "Summary" item 1 (S sinks + N window + 16 slack slots):
    every live cell has its own slot, sinks and window never share one, and a
    cell keeps its slot as the cache grows."""
    S, W, slack = 8, 40, 16
    for T in range(1, 300, 7):
        cells = o.overlay_slot_cells(T, S, W, slack)
        assert cells.shape == (S + W + slack,)
        live = [t for t in range(T) if o.overlay_live(t, T, S, W)]
        assert sorted(cells[cells >= 0].tolist()) == live
        for t in live:
            sl = o.overlay_slot(t, S, W, slack)
            assert 0 <= sl < S + W + slack and cells[sl] == t
            assert (sl < S) == (t < S)
    # the slot is a function of the cell alone
    assert o.overlay_slot(100, S, W, slack) == S + (100 - S) % (W + slack)


def test_one_shot_equals_one_append_call():
    """Appending whole groups from an empty cache in one call stores exactly
    what the one-shot encoder stores (bulk and overlay)."""
    K, V = _kv(T=128, seed=21)
    for S, W, slack in ((8, 40, 16), (0, 0, 0), (8, 64, 0), (4, 7, 3)):
        st = _run_appends(K, V, [128], S=S, W=W, slack=slack)
        kc, ks, vb, ko, vo = o.q2k_encode(K, V, 1.1, S, W, slack)
        for name, ref in (("k_codes", kc), ("k_scale", ks), ("v_blocks", vb), ("k_ovl", ko), ("v_ovl", vo)):
            assert np.array_equal(st[name], ref), (name, S, W, slack)


def test_split_appends_store_what_one_call_stores():
    """Strata #2318 "Review fixes": two-call and one-call appends store the
    same scale.  Any split of the same cells -- one cell at a time (decode),
    speculative 2-5-cell windows, 6-step writers, 100-cell prefill chunks
    that fall mid-group, a prompt of whole groups then decode -- ends in the
    same bytes, the final partial group included."""
    T = 171                                   # 5 whole groups + 11 cells
    K, V = _kv(T=T, seed=22)
    one = _run_appends(K, V, [T])
    g = np.random.default_rng(5)
    spec = []
    while sum(spec) < T:
        spec.append(int(min(g.integers(2, 6), T - sum(spec))))
    for steps in ([1] * T, [6] * (T // 6) + [T % 6], [100, 71], [64] + [1] * (T - 64), spec,
                  [33, 31, 1, 106]):
        st = _run_appends(K, V, steps)
        for name in one:
            assert np.array_equal(st[name], one[name]), (name, steps[:4])


def test_complete_groups_equal_the_one_shot_encoder():
    """Prompt + decode: once a group is complete its codes and scale are the
    one-shot encoder's, however its cells arrived."""
    K, V = _kv(T=96, seed=23)
    st = _run_appends(K, V, [40] + [1] * 56)
    kc, ks = o.q2k_encode_k(K, 1.1)
    assert np.array_equal(st["k_codes"], kc) and np.array_equal(st["k_scale"], ks)
    assert np.array_equal(st["v_blocks"], o.q2k_encode_v(V))


def test_partial_group_scale_rule():
    """The partial-group rule in closed form (Strata #2318 "Review fixes":
    s = sqrt((ss + (32 - n) prev^2) / 32), prev the previous group's scale),
    and the first group's RMS of the cells present."""
    n_kv, d = 1, 32
    a, B = 0.75, 1.1
    K = np.zeros((45, n_kv, d), np.float32)
    K[:32] = 2.0                               # group 0: RMS 2
    K[32:] = a                                 # group 1: 13 cells of a
    st = _run_appends(K, K, [45], gain=B, S=0, W=0, slack=0)
    prev = np.float32(o.f16_value(st["k_scale"][0, 0, 0])) / np.float32(B)
    s = np.sqrt((13 * a * a + 19 * float(prev) ** 2) / 32)
    got = o.f16_value(st["k_scale"][1, 0, 0]) / B
    assert abs(got - s) < 2e-3 * s
    assert st["k_scale"][0, 0, 0] == o.f16_bits(np.float32(B) * np.float32(2.0))
    # bit-exact f32 chain of the rule
    ss = np.float32(0.0)
    for _ in range(13):
        ss = np.float32(ss + np.float32(a) * np.float32(a))
    want = np.sqrt(np.float32(ss + np.float32(19) * np.float32(prev * prev)) / np.float32(32))
    assert st["k_scale"][1, 0, 0] == o.f16_bits(np.float32(B) * np.float32(want))
    # the first group, partial: RMS of its cells (7 cells of 3.0 -> 3.0)
    K0 = np.full((7, n_kv, d), 3.0, np.float32)
    st0 = _run_appends(K0, K0, [7], gain=B, S=0, W=0, slack=0)
    assert st0["k_scale"][0, 0, 0] == o.f16_bits(np.float32(B) * np.float32(3.0))
    # absent cells of a partial group carry code 0
    st1 = _run_appends(K[:40], K[:40], [40], gain=B, S=0, W=0, slack=0)
    packed = st1["k_codes"][1, 0, 0]
    codes = [(int(packed[j // 4]) >> (2 * (j % 4))) & 3 for j in range(32)]
    assert all(c == 0 for c in codes[8:])


def test_writers_agree_and_decode_reads_the_ring():
    """Single-cell, 6-step and batch overlay writers leave the same slots
    (Strata #2318 "Review fixes"); the decoded cache reads every live cell's
    fp16 copy from its ring slot and every other cell from the bulk."""
    T, S, W, slack = 150, 8, 40, 16
    K, V = _kv(T=T, seed=24)
    a = _run_appends(K, V, [1] * T, S=S, W=W, slack=slack)
    b = _run_appends(K, V, [6] * 25, S=S, W=W, slack=slack)
    c = _run_appends(K, V, [T], S=S, W=W, slack=slack)
    for name in ("k_ovl", "v_ovl"):
        assert np.array_equal(a[name], c[name]) and np.array_equal(b[name], c[name])
    Kd, Vd = o.q2k_decode(c["k_codes"], c["k_scale"], c["v_blocks"], c["k_ovl"], c["v_ovl"],
                          S, W, slack, T)
    Kb, Vb = o.q2k_decode(c["k_codes"], c["k_scale"], c["v_blocks"], None, None, S, W, slack, T)
    for t in range(T):
        if o.overlay_live(t, T, S, W):
            assert np.array_equal(Kd[t], K[t].astype(np.float16).astype(np.float64))
            assert np.array_equal(Vd[t], V[t].astype(np.float16).astype(np.float64))
        else:
            assert np.array_equal(Kd[t], Kb[t]) and np.array_equal(Vd[t], Vb[t])


def _f16_from_bits(bits: int) -> float:
    # IEEE binary16 value through the struct module (independent of numpy's
    # float16 path the oracle uses)
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def test_bulk_k_decode_is_level_times_stored_scale():
    """Strata #2318 "Summary" item 3 and "Measurements" (the K-gain pin): a
    bulk K cell reads back as level[code] times the stored fp16 scale, which
    already carries B (the codes were chosen against the un-gained rule).
    The 2-bit codes are unpacked here by an own loop over the byte layout
    (cell j of a 32-cell group in bits 2*(j%4) of byte j//4 of its channel),
    so a wrong cell order or a scale divided by B in the oracle's decode
    fails."""
    T, n_kv, d = 96, 2, 64
    K, _ = _kv(T=T, n_kv=n_kv, d=d, seed=21)
    G = T // 32
    lv = o.codebook_f16(4)
    # the 4 levels: ascending, symmetric, Max (1960) Table I to its 4 digits
    row = next(s for s in lines("max1960_gaussian_levels.txt") if s.split()[0] == "4")
    max1960 = [float(t) for t in row.split(";")[0].split()[1:]]
    assert np.all(np.diff(lv) > 0) and np.array_equal(lv, -lv[::-1])
    assert np.allclose(lv[2:], max1960, atol=1e-3)
    vb0 = np.zeros((T, n_kv, d // 32, 18), np.uint8)
    dec = {}
    for B in (1.0, 1.10, 2.0):
        kc, ks = o.q2k_encode_k(K, B)
        Kd, _ = o.q2k_decode(kc, ks, vb0, None, None, 0, 0)
        for g in range(G):
            for h in range(n_kv):
                for c in range(d):
                    scale = _f16_from_bits(ks[g, h, c])
                    for j in range(32):
                        code = (int(kc[g, h, c, j // 4]) >> (2 * (j % 4))) & 3
                        assert Kd[g * 32 + j, h, c] == float(lv[code]) * scale, (B, g, h, c, j)
        dec[B] = (Kd, ks)
    # B = 2 doubles every cell whose stored scale is a normal fp16 number
    Kd1, ks1 = dec[1.0]
    Kd2, _ = dec[2.0]
    normal = np.repeat(((ks1 & 0x7C00) != 0)[:, None], 32, axis=1).reshape(T, n_kv, d)
    assert normal.mean() > 0.9
    assert np.array_equal(Kd2[normal], 2.0 * Kd1[normal])
    # B = 1.10: the decoded cell over the stored scale is the level nearest
    # to k / rule, the rule being the group RMS (f64 here)
    Kd11, ks11 = dec[1.10]
    rms = np.sqrt(np.mean(K.astype(np.float64).reshape(G, 32, n_kv, d) ** 2, axis=1))
    z = K.astype(np.float64).reshape(G, 32, n_kv, d) / rms[:, None]
    dist = np.abs(z[..., None] - lv.astype(np.float64))
    srt = np.sort(dist, -1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-5
    stored = np.vectorize(_f16_from_bits)(ks11)[:, None].repeat(32, axis=1)
    level_read = Kd11.reshape(G, 32, n_kv, d) / stored
    assert np.array_equal(level_read[clear], lv.astype(np.float64)[np.argmin(dist, -1)][clear])
