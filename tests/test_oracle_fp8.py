"""Pins for the oracle's fp8 e4m3 decode and KV8 row encoder (CPU only).

Each check ties the oracle to something other than itself: the decode rule the
page prints (golden fixture), torch's float8_e4m3fn conversions (an
independent library routine), brute-force nearest-value search, and
invariants of the amax/448 scale.
"""
import numpy as np
import pytest
import torch

from oracle import kvq_oracle as o
from tests._golden import lines, page_numbers
from synth import edge_rows


def test_decode_matches_page_rule_fixture():
    # colibri #399, rebase comment "3. HIP portability"
    lut = o.e4m3_table()
    n = 0
    for s in lines("e4m3_values.txt"):
        code, val = s.split()
        assert lut[int(code, 16)] == float(val), code
        n += 1
    assert n >= 15


def test_decode_matches_torch_float8_e4m3fn():
    lut = o.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for b in range(256):
        if b in (0x7F, 0xFF):
            assert np.isnan(ref[b]) and lut[b] == 0.0      # the page reads NaN back as 0
        else:
            assert lut[b] == ref[b], hex(b)


def test_exhaustive_round_trip_and_midpoints():
    # test_kv_fp8 on colibri #399 "Validation": exhaustive e4m3 round trip + RNE
    lut = o.e4m3_table()
    pos = lut[:0x7F]                                   # 0x00..0x7E, increasing
    assert np.all(np.diff(pos) > 0)
    codes = np.arange(0x7F)
    got = o.e4m3_rne_magnitude(pos.astype(np.float32))
    assert np.array_equal(got, codes)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # midpoints exact in f32
    want = np.where(codes[:-1] % 2 == 0, codes[:-1], codes[1:])             # ties -> even code
    assert np.array_equal(o.e4m3_rne_magnitude(mids), want)
    below = np.nextafter(mids, np.float32(0))
    above = np.nextafter(mids, np.float32(1e9))
    assert np.array_equal(o.e4m3_rne_magnitude(below), codes[:-1])
    assert np.array_equal(o.e4m3_rne_magnitude(above), codes[1:])


def _nearest_code_bruteforce(a):
    pos = o.e4m3_table()[:0x7F]
    a = a.astype(np.float64)
    i = np.clip(np.searchsorted(pos, a), 1, 0x7E)
    lo, hi = pos[i - 1], pos[i]
    dl, dh = a - lo, hi - a
    pick = np.where(dl < dh, i - 1, np.where(dh < dl, i, np.where((i - 1) % 2 == 0, i - 1, i)))
    pick = np.where(a >= pos[-1], 0x7E, pick)
    pick = np.where(a <= 0, 0, pick)
    return pick.astype(np.uint8)


def test_rne_bruteforce_random_and_structured():
    g = np.random.default_rng(5)
    a = np.concatenate([
        g.uniform(0, 460, 300000),
        np.exp(g.uniform(np.log(1e-6), np.log(448), 300000)),
        g.uniform(0, 2.0 ** -6, 100000),
        np.array([0.0, 448.0, 449.0, 463.9, 464.0, 1e30, 2.0 ** -10, 2.0 ** -149]),
    ]).astype(np.float32)
    assert np.array_equal(o.e4m3_rne_magnitude(a), _nearest_code_bruteforce(a))


def test_rne_matches_torch_in_range():
    g = np.random.default_rng(6)
    a = np.concatenate([g.uniform(0, 448, 500000),
                        np.exp(g.uniform(np.log(1e-7), np.log(448), 500000))]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(o.e4m3_rne_magnitude(a), ref)


def test_kv8_encode_invariants():
    g = np.random.default_rng(7)
    x = (g.standard_normal((300, 512)) * np.exp(g.standard_normal(512))).astype(np.float32)
    x = np.concatenate([x, edge_rows(512)])
    codes, scale = o.kv8_encode(x)
    amax = np.max(np.abs(x), axis=1)
    live = amax > 0
    # scale = amax/448 in f32 (the page's per-row scale)
    assert np.array_equal(scale[live], (amax[live] / np.float32(448)).astype(np.float32))
    # the amax element always lands on +-448 (0x7E / 0xFE)
    for r in np.nonzero(live & (scale > 2.0 ** -126))[0]:
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] & 0x7F == 0x7E
        assert (codes[r, j] >> 7) == (1 if x[r, j] < 0 else 0)
    # zero row: scale 0, codes 0
    assert np.all(codes[~live] == 0) and np.all(scale[~live] == 0)
    # no NaN code is ever produced
    assert not np.any((codes & 0x7F) == 0x7F)
    # decode error within half an e4m3 step (relative 2^-4) or half a subnormal step
    xh = o.kv8_decode(codes, scale)
    ok = live & (scale > 2.0 ** -126)
    err = np.abs(xh[ok] - x[ok])
    bound = np.maximum(np.abs(x[ok]) * 2.0 ** -4, scale[ok, None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_kv8_sign_of_underflow_kept():
    x = np.zeros((1, 8), np.float32)
    x[0, 0] = 448.0
    x[0, 1] = -1e-5          # rounds to zero magnitude, keeps the sign bit
    x[0, 2] = -0.0
    codes, scale = o.kv8_encode(x)
    assert scale[0] == 1.0
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0x80 and codes[0, 2] == 0x80 and codes[0, 3] == 0x00


def test_kv8_byte_accounting_matches_page_ratio():
    ratio = 512 * 4 / o.row_bytes("fp8", 512)
    assert o.row_bytes("fp8", 512) == 516
    assert abs(ratio - page_numbers()["kv8_vs_f32_ratio"]) < 0.1


def test_kv8_subnormal_scale_rows_saturate():
    """Rows whose amax is an f32 subnormal near 2^-149 * 448 get a coarse
    subnormal scale, so quotients x / scale reach about 667.  Reading C-4 of
    the encoder (colibri #399 "Commits" item 1, 448 the largest e4m3 value):
    every quotient at or above 448 saturates to 0x7E / 0xFE; below it the
    byte is the RNE nearest code (brute force), and no NaN code appears."""
    from synth import tiny_amax_rows
    x = tiny_amax_rows(64)
    codes, scale = o.kv8_encode(x)
    live = scale > 0
    assert live.sum() >= 60 and np.all(codes[~live] == 0)
    q = np.abs(x[live] / scale[live, None]).astype(np.float32)       # one f32 divide each
    assert q.max() > 600                                              # the case is reached
    mag = codes[live] & 0x7F
    assert np.all(mag[q >= 448] == 0x7E)
    assert np.array_equal(mag, _nearest_code_bruteforce(q.ravel()).reshape(q.shape))
    assert not np.any(mag == 0x7F)
    sign = codes[live] >> 7
    assert np.array_equal(sign, np.signbit(x[live]).astype(np.uint8))
