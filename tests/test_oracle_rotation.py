"""Pins for the oracle's rotation pieces: SplitMix64 signs, FWHT, codebooks."""
import math
import struct

import numpy as np
import pytest

from oracle import kvq_oracle as o
from tests._golden import lines


def test_splitmix64_published_outputs():
    # Reference outputs of SplitMix64 from state 0 (the published generator's
    # first three outputs, as used to seed xoshiro generators).
    assert o.splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_rotation_signs_are_pm1_and_square_to_identity():
    d = o.rotation_signs(0x1234, 512)
    assert set(np.unique(d)) <= {-1.0, 1.0}
    assert np.array_equal(d * d, np.ones(512, np.float32))
    # bit i of word i//64 decides sign i
    w = o.splitmix64(0x1234, 8)
    for i in (0, 1, 63, 64, 200, 511):
        assert (d[i] < 0) == bool((w[i // 64] >> (i % 64)) & 1)
    # roughly balanced
    assert 200 < np.sum(d < 0) < 312


def _sylvester(n):
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 64, 128])
def test_fwht_equals_sylvester_matrix(n):
    g = np.random.default_rng(n)
    v = g.integers(-50, 50, size=(5, n)).astype(np.float32)
    H = _sylvester(n)
    assert np.array_equal(o.fwht_f32(v).astype(np.float64), v.astype(np.float64) @ H.T)
    assert np.array_equal(o.fwht_f64(v), v.astype(np.float64) @ H.T)


@pytest.mark.parametrize("n", [2, 32, 512, 1024])
def test_fwht_self_inverse(n):
    # test_kv_tq on colibri #399 "Validation": rotation self-inverse
    g = np.random.default_rng(n)
    v = g.integers(-1000, 1000, size=(4, n)).astype(np.float32)
    assert np.array_equal(o.fwht_f32(o.fwht_f32(v)), v * np.float32(n))


def test_fwht_float_rounding_within_bound():
    g = np.random.default_rng(3)
    v = g.standard_normal((16, 512)).astype(np.float32)
    exact = v.astype(np.float64) @ _sylvester(512).T
    err = np.abs(o.fwht_f32(v) - exact)
    # 9 stages of one rounding each: relative to sum|v| the error is < 9 * 2^-24
    assert np.all(err <= 9 * 2.0 ** -24 * np.sum(np.abs(v), axis=1, keepdims=True))


def test_codebooks_match_max_1960_table():
    for s in lines("max1960_gaussian_levels.txt"):
        left, mse = s.split(";")
        parts = left.split()
        L = int(parts[0])
        pos = [float(t) for t in parts[1:]]
        c, D = o.lloyd_max_gaussian(L)
        assert np.allclose(c[L // 2:], pos, atol=6e-4), (L, c)
        assert np.allclose(-c[:L // 2][::-1], pos, atol=6e-4)
        assert abs(D - float(mse)) < 1e-3 * float(mse)   # table printed to 4 figures


def test_codebooks_satisfy_lloyd_conditions():
    from scipy.integrate import quad
    for L in (4, 16):
        c, D = o.lloyd_max_gaussian(L)
        b = np.concatenate([[-np.inf], (c[:-1] + c[1:]) / 2, [np.inf]])
        phi = lambda z: math.exp(-z * z / 2) / math.sqrt(2 * math.pi)
        for k in range(L):
            num = quad(lambda z: z * phi(z), b[k], b[k + 1], epsabs=1e-14)[0]
            den = quad(phi, b[k], b[k + 1], epsabs=1e-14)[0]
            assert abs(num / den - c[k]) < 1e-9
        mse = sum(quad(lambda z, k=k: (z - c[k]) ** 2 * phi(z), b[k], b[k + 1], epsabs=1e-14)[0]
                  for k in range(L))
        assert abs(mse - D) < 1e-9


def test_codebook_f16_rounding_is_nearest():
    for L in (4, 16):
        c, _ = o.lloyd_max_gaussian(L)
        cb = o.codebook_f16(L)
        for x, y in zip(c, cb):
            ref = struct.unpack("<e", struct.pack("<e", float(x)))[0]   # Python's own RNE to half
            assert y == ref
        assert np.array_equal(cb, -cb[::-1])                           # symmetric
        tau = o.codebook_thresholds(L)
        assert np.array_equal(tau.astype(np.float64), (cb[:-1].astype(np.float64) + cb[1:]) / 2)
        assert tau[L // 2 - 1] == 0.0


def test_f16_conversion_matches_python_struct():
    g = np.random.default_rng(9)
    a = np.concatenate([g.standard_normal(20000) * 10, g.standard_normal(5000) * 1e-5,
                        np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -25, 3 * 2 ** -25, 65504.0, 65519.0])])
    a = a.astype(np.float32)
    bits = o.f16_bits(a)
    ref = np.array([struct.unpack("<H", struct.pack("<e", float(v)))[0] for v in a], np.uint16)
    assert np.array_equal(bits, ref)
