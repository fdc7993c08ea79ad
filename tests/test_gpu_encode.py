"""GPU encoders vs the oracle: every stored byte must be identical.

Inputs come from the seeded generators in synth/ (shapes and distributions of
the workloads: the MLA latent rows with lognormal channel gains, Strata's
2 x 256 GQA K/V with sigma 1.5 gains), plus edge rows and ragged / small
widths.  Full-size cases run at the sizes the benchmark uses; the TQ4 128k
case compares a random sample of rows (the encoder is row-independent).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import kvq_oracle as o
from tests._gpu import DEV, assert_bytes_equal, dev, host, host_u16, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_kv_cache_e4m3_amd as kq


def _fp8_case(x, what):
    say(f"kv_encode_fp8 {what} shape={x.shape}")
    codes, scales = kq.kv_encode_fp8(dev(x))
    wc, ws = o.kv8_encode(x)
    assert_bytes_equal(host(codes), wc, f"fp8 codes {what}")
    assert_bytes_equal(host(scales), ws, f"fp8 scales {what}")


def test_fp8_tiny_workload():
    x, _ = synth.latent_inputs(synth.WORKLOADS["tiny_kv8"])
    _fp8_case(x, "tiny 256x64")


def test_fp8_mla_workload_full():
    x, _ = synth.latent_inputs(synth.WORKLOADS["kv8_decode"])
    _fp8_case(x, "kv8_decode 32768x512")


@pytest.mark.parametrize("d", [8, 64, 512, 1024, 4096])
def test_fp8_edge_rows(d):
    _fp8_case(synth.edge_rows(d), f"edge d={d}")


@pytest.mark.parametrize("d", [1, 3, 100, 520, 4104])
def test_fp8_ragged_widths(d):
    g = np.random.default_rng(d)
    x = (g.standard_normal((37, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    _fp8_case(x, f"ragged d={d}")


def test_fp8_unaligned_append_and_empty():
    g = np.random.default_rng(1)
    x = g.standard_normal((10, 64)).astype(np.float32)
    xbuf = torch.zeros((10 * 64 + 1,), dtype=torch.float32, device=DEV)
    xbuf[1:] = dev(x).reshape(-1)
    cbuf = torch.zeros((10 * 64 + 5,), dtype=torch.uint8, device=DEV)
    scales = torch.zeros((12,), dtype=torch.float32, device=DEV)
    say("kv_encode_fp8 rows at 4-byte-aligned x and 1-byte-aligned codes")
    st = kq.lib.kv_encode_fp8(xbuf[1:].data_ptr(), 10, 64, cbuf[5:].data_ptr(), scales[2:].data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert st == 0
    wc, ws = o.kv8_encode(x)
    assert_bytes_equal(host(cbuf)[5:].reshape(10, 64), wc, "append codes")
    assert_bytes_equal(host(scales)[2:], ws, "append scales")
    assert np.all(host(cbuf)[:5] == 0) and np.all(host(scales)[:2] == 0)
    say("kv_encode_fp8 n_rows=0")
    assert kq.lib.kv_encode_fp8(xbuf.data_ptr(), 0, 64, cbuf.data_ptr(), scales.data_ptr(), None) == 0


def _rounding_points() -> np.ndarray:
    """Every e4m3 magnitude, every midpoint between adjacent magnitudes, and the
    float32 values 1 and 2 ulps either side of each; half the smallest e4m3
    subnormal and its neighbours; a few values far below it.  All in [0, 448]."""
    tab = o.e4m3_table()
    mags = np.unique(np.abs(tab))
    mids = (mags[:-1] + mags[1:]) / 2.0                   # exact in float32
    base = np.concatenate([mags, mids, [2.0 ** -10, 2.0 ** -11, 1e-30, 1e-40]]).astype(np.float32)
    bits = base.view(np.uint32).astype(np.int64)
    near = [bits + k for k in (-2, -1, 0, 1, 2)]
    vals = np.concatenate(near)
    vals = vals[(vals >= 0) & (vals <= np.float32(448.0).view(np.uint32))].astype(np.uint32).view(np.float32)
    return np.unique(vals)


def test_fp8_rounding_points():
    """Rows whose largest magnitude is 448 have scale 448/448 = 1 exactly, so
    each element's quotient is the element itself: the codes of every e4m3
    value, every rounding midpoint and their float32 neighbours, with both
    signs (negative zero included), equal the oracle's round-to-nearest-even."""
    v = _rounding_points()
    v = np.concatenate([v, -v])
    per_row = 511
    n_rows = (v.size + per_row - 1) // per_row
    x = np.zeros((n_rows, 512), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(n_rows * per_row, np.float32)
    flat[:v.size] = v
    x[:, 1:] = flat.reshape(n_rows, per_row)
    say(f"kv_encode_fp8 rounding points: {v.size} values in {n_rows} rows")
    codes, scales = kq.kv_encode_fp8(dev(x))
    assert np.all(host(scales) == 1.0)
    wc, _ = o.kv8_encode(x)
    assert_bytes_equal(host(codes), wc, "fp8 codes at the rounding points")
    # the same values through the general (any width) path
    xr = np.ascontiguousarray(x[:, :509])
    say("kv_encode_fp8 rounding points, d=509")
    codes_r, _ = kq.kv_encode_fp8(dev(xr))
    assert_bytes_equal(host(codes_r), o.kv8_encode(xr)[0], "fp8 codes at the rounding points, d=509")


def _tq4_case(x, what, sample=None):
    say(f"kv_encode_tq4 {what} shape={x.shape}")
    packed, radius = kq.kv_encode_tq4(dev(x), synth.ROT_SEED)
    gp, gr = host(packed), host(radius)
    rows = np.arange(x.shape[0]) if sample is None else sample
    wp, wr = o.tq4_encode(x[rows], synth.ROT_SEED)
    assert_bytes_equal(gp[rows], wp, f"tq4 packed {what}")
    assert_bytes_equal(gr[rows], wr, f"tq4 radius {what}")


@pytest.mark.parametrize("d", [2, 4, 8, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_tq4_widths(d):
    g = np.random.default_rng(d + 5)
    x = (g.standard_normal((70, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    _tq4_case(x, f"d={d}")


@pytest.mark.parametrize("d", [64, 512])
def test_tq4_edge_rows(d):
    _tq4_case(synth.edge_rows(d), f"edge d={d}")


def test_tq4_mla_workload_full_size_sampled():
    w = synth.WORKLOADS["tq4_decode"]
    x, _ = synth.latent_inputs(w)
    sample = np.sort(np.random.default_rng(0).choice(w.T, 6000, replace=False))
    sample = np.concatenate([[0, 1, w.T - 1], sample])
    _tq4_case(x, "tq4_decode 131072x512", sample=sample)


def test_tq4_512_output_4_byte_aligned():
    """d = 512 rows packed into a buffer that starts 4 bytes past a 16-byte
    boundary (the encoder's narrow-store path), a ragged row count, and the
    bytes around the destination left untouched."""
    g = np.random.default_rng(41)
    x = (g.standard_normal((37, 512)) * np.exp(g.standard_normal(512))).astype(np.float32)
    n = x.shape[0]
    buf = torch.zeros(n * 256 + 8, dtype=torch.uint8, device=DEV)
    rad = torch.empty(n, dtype=torch.float32, device=DEV)
    dst = buf[4:4 + n * 256]
    assert dst.data_ptr() % 16 == 4
    xd = dev(x)
    say("kv_encode_tq4 d=512 into a 4-byte-aligned destination")
    st = kq.lib.kv_encode_tq4(xd.data_ptr(), n, 512, synth.ROT_SEED, dst.data_ptr(), rad.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert st == 0
    wp, wr = o.tq4_encode(x, synth.ROT_SEED)
    got = host(buf)
    assert_bytes_equal(got[4:4 + n * 256].reshape(n, 256), wp, "tq4 packed at +4 bytes")
    assert_bytes_equal(host(rad), wr, "tq4 radius")
    assert np.all(got[:4] == 0) and np.all(got[4 + n * 256:] == 0)


def test_tq4_seed_changes_bytes():
    x = np.random.default_rng(3).standard_normal((8, 256)).astype(np.float32)
    say("kv_encode_tq4 two seeds")
    a, _ = kq.kv_encode_tq4(dev(x), 1)
    b, _ = kq.kv_encode_tq4(dev(x), 2)
    assert not np.array_equal(host(a), host(b))
    assert_bytes_equal(host(b), o.tq4_encode(x, 2)[0], "tq4 seed 2")


def _q2k_case(K, V, gain, ns, nw, what):
    say(f"kv_encode_q2k {what} K={K.shape} gain={gain} sink={ns} window={nw}")
    enc = kq.kv_encode_q2k(dev(K), dev(V), gain, ns, nw)
    kc, ks, vb, ko, vo = o.q2k_encode(K, V, gain, ns, nw)
    assert_bytes_equal(host(enc["k_codes"]), kc, f"q2k k_codes {what}")
    assert_bytes_equal(host_u16(enc["k_scale"]), ks, f"q2k k_scale {what}")
    assert_bytes_equal(host(enc["v_blocks"]), vb, f"q2k v_blocks {what}")
    if ns + nw > 0:
        assert_bytes_equal(host_u16(enc["k_ovl"]), ko, f"q2k k_ovl {what}")
        assert_bytes_equal(host_u16(enc["v_ovl"]), vo, f"q2k v_ovl {what}")


def test_q2k_workload_full():
    w = synth.WORKLOADS["q2k_decode"]
    K, V, _ = synth.q2k_inputs(w)
    _q2k_case(K, V, w.k_gain, w.n_sink, w.n_window, "q2k_decode 32768x2x256")


@pytest.mark.parametrize("T,n_kv,d,ns,nw", [(32, 1, 32, 0, 0), (64, 2, 64, 8, 16), (96, 3, 96, 4, 90),
                                             (32, 2, 512, 8, 256), (128, 1, 256, 0, 32)])
def test_q2k_shapes_and_overlays(T, n_kv, d, ns, nw):
    g = np.random.default_rng(T * 7 + d)
    K = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    V = (g.standard_normal((T, n_kv, d)) * np.exp(1.5 * g.standard_normal((n_kv, d)))).astype(np.float32)
    _q2k_case(K, V, 1.10, ns, nw, f"T={T}")


def test_q2k_edge_values():
    g = np.random.default_rng(11)
    K = g.standard_normal((64, 2, 64)).astype(np.float32)
    V = g.standard_normal((64, 2, 64)).astype(np.float32)
    K[:32, 0, :] = 0.0                       # a zero group -> codes 0, scale 0
    V[3, 1, :32] = 0.0                       # a zero block -> d 0, codes 8
    V[4, 0, :32] = 1e-6                      # d underflows to an fp16 subnormal
    K[40:, 1, 5] = 1e-4                      # tiny constant channel
    V[7, 0, 32:] = np.linspace(-7, 7, 32)    # exact ties of x/d
    _q2k_case(K, V, 1.10, 2, 3, "edge values")
    _q2k_case(K, V, 1.0, 0, 0, "edge values, no gain, no overlay")


@pytest.mark.parametrize("d", [8, 100, 512])
def test_fp8_subnormal_scale_saturation(d):
    """Rows with amax in [3e-43, 1.3e-42]: subnormal scales, quotients up to
    about 667, which must store the saturated 0x7E / 0xFE (never the NaN code);
    d = 512 and 8 take the vector encoder, d = 100 the any-width one."""
    x = synth.tiny_amax_rows(d)
    _fp8_case(x, f"subnormal-scale rows d={d}")
    codes, _ = o.kv8_encode(x)
    assert np.any(codes == 0x7E) and np.any(codes == 0xFE)
