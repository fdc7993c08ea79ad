"""Pins for the oracle's rotated-int4 (TQ4) codec."""
import numpy as np
import pytest

from oracle import kvq_oracle as o
from tests._golden import page_numbers

SEED = 0x5EED000000000003


def _H(n):
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_radius_small_exact_cases():
    x = np.array([[3, 4], [0, 0], [-3, 4]], np.float32)
    assert np.array_equal(o.tq4_radius(x), np.array([5, 0, 5], np.float32))
    x = np.array([[1, 2, 2, 4]], np.float32)
    assert o.tq4_radius(x)[0] == 5.0


def test_radius_close_to_f64_norm():
    g = np.random.default_rng(1)
    x = g.standard_normal((100, 512)).astype(np.float32)
    r = o.tq4_radius(x).astype(np.float64)
    ref = np.linalg.norm(x.astype(np.float64), axis=1)
    assert np.all(np.abs(r - ref) <= 12 * 2.0 ** -24 * ref)


def test_orthogonality_identities():
    # colibri #399 "Ready for review" comment: q . x_hat == rotate(q) . c and
    # sum_t w_t x_hat_t == unrotate(sum_t w_t c_t), checked in f64 against an
    # explicit Sylvester matrix (independent of the FWHT code).
    n = 128
    g = np.random.default_rng(2)
    x = (g.standard_normal((40, n)) * np.exp(g.standard_normal(n))).astype(np.float32)
    packed, r = o.tq4_encode(x, SEED)
    xh = o.tq4_decode(packed, r, SEED)
    c = o.codebook_f16(16).astype(np.float64)[o.tq4_unpack(packed)]
    D = np.diag(o.rotation_signs(SEED, n).astype(np.float64))
    H = _H(n)
    q = g.standard_normal(n)
    qrot = H @ D @ q
    lhs = xh @ q
    rhs = (r.astype(np.float64) / n) * (c @ qrot)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    w = g.random(40)
    ctx = w @ xh
    ctx_rot = (w * r.astype(np.float64)) @ c
    assert np.allclose(ctx, D @ H @ ctx_rot / n, rtol=1e-12, atol=1e-12)
    # and decode is the exact inverse rotation of the scaled levels
    assert np.allclose(xh, (r[:, None] / n) * (c @ H.T @ D), rtol=1e-12, atol=1e-12)


def test_distortion_matches_page():
    # colibri #399 "Why rotated-int4 for the 4-bit tier": ~0.096 rel-L2 at 4 bits
    g = np.random.default_rng(3)
    x = g.standard_normal((3000, 512)).astype(np.float32)
    packed, r = o.tq4_encode(x, SEED)
    xh = o.tq4_decode(packed, r, SEED)
    rel = np.linalg.norm(xh - x) / np.linalg.norm(x)
    page = page_numbers()["tq4_rel_l2"]
    assert abs(rel - page) < 0.003, rel
    # the Gaussian closed form sqrt(D16) bounds it from the same side
    _, D = o.lloyd_max_gaussian(16)
    assert abs(rel - np.sqrt(D)) < 0.003


def test_levels_are_nearest_codebook_values():
    g = np.random.default_rng(4)
    x = g.standard_normal((200, 256)).astype(np.float32)
    packed, r = o.tq4_encode(x, SEED)
    idx = o.tq4_unpack(packed)
    y = (x.astype(np.float64) * o.rotation_signs(SEED, 256)) @ _H(256).T
    z = y / r[:, None].astype(np.float64)
    cb = o.codebook_f16(16).astype(np.float64)
    dist = np.abs(z[..., None] - cb[None, None, :])
    best = np.argmin(dist, axis=-1)
    margin = np.sort(dist, axis=-1)[..., 1] - np.sort(dist, axis=-1)[..., 0]
    clear = margin > 1e-5                       # away from a decision boundary
    assert np.array_equal(idx[clear], best[clear])
    assert clear.mean() > 0.99


def test_inert_rows_and_refusals():
    x = np.zeros((2, 64), np.float32)
    packed, r = o.tq4_encode(x, SEED)
    assert np.all(packed == 0) and np.all(r == 0)
    assert np.all(o.tq4_decode(packed, r, SEED) == 0)
    # colibri #553 rebase comment: non-power-of-two widths are refused
    with pytest.raises(ValueError):
        o.tq4_encode(np.ones((1, 96), np.float32), SEED)


def test_nibble_order():
    x = np.zeros((1, 4), np.float32)
    x[0] = [1.0, 0.0, 0.0, 0.0]
    packed, r = o.tq4_encode(x, 0)
    idx = o.tq4_unpack(packed)
    assert packed[0, 0] == (idx[0, 0] | (idx[0, 1] << 4))
    assert packed.shape == (1, 2)


def test_tq4_byte_accounting_matches_page_ratio():
    assert o.row_bytes("tq4", 512) == 260
    assert abs(512 * 4 / o.row_bytes("tq4", 512) - page_numbers()["tq4_vs_f32_ratio"]) < 0.1
