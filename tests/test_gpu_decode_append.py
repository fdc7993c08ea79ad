"""attn_decode_append_fp8: one KV8 decode step whose new row is encoded by the
same call ([colibri #399] "Summary" / "Commits" item 1 for the row, "Ready for
review" comment for the decode).

The call must leave exactly the bytes kv_encode_fp8 writes for that row (the
oracle's bytes, checked first), and its output and lse must equal, bit for
bit, those of attn_decode_quant over the cache the encoder wrote: the fused
launch decodes the same values in the same order.  Before each call the new
row's slot holds other bytes (NaN codes and a huge scale), so a read of the
stale row anywhere in the decode would show.  One case is also held to the
oracle's attention bar directly.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import kvq_oracle as o
from tests._gpu import assert_bytes_equal, check_attention, dev, host, reference, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_kv_cache_e4m3_amd as kq


def _inputs(T, H, d, seed, last):
    w = synth.Workload("append", "fp8", T=T, Hq=H, d=d, sigma=1.0, seed=seed)
    x, q = synth.latent_inputs(w)
    if last == "large":
        x[-1] *= 1000.0                 # the new row carries the chunk's largest scale
    elif last == "zero":
        x[-1] = 0.0                     # scale 0, all-zero codes
    elif last == "subnormal":
        x[-1] *= 1e-43                  # subnormal scale, saturating quotients
    return x, q, w.sm_scale


def _run(T, H, d=512, seed=7, last="plain", rope=False):
    x, q, sm = _inputs(T, H, d, seed, last)
    say(f"append decode T={T} H={H} d={d} last={last} rope={rope}")
    xd = dev(x)
    codes, scales = kq.kv_encode_fp8(xd)
    wc, wsc = o.kv8_encode(x[-1:])
    assert_bytes_equal(host(codes)[-1:], wc, "encoder codes of the new row")
    assert_bytes_equal(host(scales)[-1:], wsc, "encoder scale of the new row")
    rope_parts = None
    if rope:
        xr = synth.gained_rows(synth.rng(seed + 1), T, 64, 1.0)
        rope_parts = kq.kv_encode_fp8(dev(xr))
        q = np.concatenate([q, synth.rng(seed + 2).standard_normal((H, 64), dtype=np.float32)], axis=1)
    qd = dev(q)
    ref = kq.Cache.fp8(codes, scales, rope=rope_parts)
    out0, lse0 = kq.attn_decode_quant(ref, qd, sm)

    codes2, scales2 = codes.clone(), scales.clone()
    codes2[-1] = 0x7F                   # e4m3 NaN
    scales2[-1] = 3.0e38
    cache = kq.Cache.fp8(codes2, scales2, rope=rope_parts)
    out1, lse1 = kq.attn_decode_append_fp8(cache, xd[-1], qd, sm)
    assert_bytes_equal(host(codes2), host(codes), "codes after the step")
    assert_bytes_equal(host(scales2), host(scales), "scales after the step")
    o0, o1, l0, l1 = host(out0), host(out1), host(lse0), host(lse1)
    assert np.array_equal(o1.view(np.uint32), o0.view(np.uint32)), \
        f"out differs from encode + decode in {np.count_nonzero(o1 != o0)} elements"
    assert np.array_equal(l1.view(np.uint32), l0.view(np.uint32)), "lse differs from encode + decode"
    return x, q, sm, o1, l1


@pytest.mark.parametrize("T,H,last", [
    (32768, 64, "plain"),       # the MLA decode shape: 4 tile rounds per workgroup
    (1000, 64, "large"),        # one round: the new row sits in the first prefetch
    (40500, 256, "plain"),      # 2560-row chunks: the new row past the first 2048 row factors
    (300, 16, "zero"),
    (300, 16, "subnormal"),
    (257, 5, "large"),          # a partial head group
    (1, 16, "plain"),           # the new row is the whole cache
])
def test_append_decode_matches_encode_then_decode(T, H, last):
    _run(T, H, last=last)


@pytest.mark.parametrize("T,H,d,rope", [
    (256, 4, 64, False),        # general path: the encoder runs first
    (3000, 64, 512, True),      # a rope part: per-head-group kernel without the fused row
    (200001, 64, 512, False),   # 64-head shared-tile decode
])
def test_append_decode_unfused_paths(T, H, d, rope):
    _run(T, H, d=d, rope=rope)


def test_append_decode_against_oracle():
    x, q, sm, out, lse = _run(4000, 64, last="large")
    xh = o.kv8_decode(*o.kv8_encode(x))
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, sm)
    check_attention(out, lse, ro, rl, "append decode T=4000 H=64", twin=tw)

