"""attn_decode_quant_noalloc (the decode without a workspace, for callers that
cannot allocate) against attn_decode_quant through the C ABI: the same
kernels and plan, so the outputs must be identical -- on calls in a row over
one GPU's shared scratch, each later call smaller than the first, and within
the attention bar of the float64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from oracle import kvq_oracle as o
from tests._gpu import DEV, check_attention, dev, host, reference, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import quantized_kv_cache_e4m3_amd as kq


def _both(cache, q, sm_scale, what):
    qd = dev(q)
    Hq, d = q.shape[0], cache.d
    out_ws = torch.full((Hq, d), 7.0, dtype=torch.float32, device=DEV)
    lse_ws = torch.full((Hq,), 7.0, dtype=torch.float32, device=DEV)
    out_na = torch.full((Hq, d), -7.0, dtype=torch.float32, device=DEV)
    lse_na = torch.full((Hq,), -7.0, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    say(f"attn_decode_quant {what}")
    kq.attn_decode_quant(cache, qd, sm_scale, out=out_ws, lse=lse_ws)
    say(f"attn_decode_quant_noalloc {what}")
    st = kq.lib.attn_decode_quant_noalloc(cache.ref, qd.data_ptr(), Hq, float(sm_scale), out_na.data_ptr(),
                                          lse_na.data_ptr(), stream)
    assert st == 0, kq.kvq_status_str(st)
    a, la, b, lb = host(out_ws), host(lse_ws), host(out_na), host(lse_na)
    assert np.array_equal(a, b) and np.array_equal(la, lb), what
    return b, lb


def test_noalloc_equals_workspace_decode_calls_in_a_row():
    # 1: the KV8 decode workload (T=32768, 64 heads: 64 chunks of partials)
    w = synth.WORKLOADS["kv8_decode"]
    x, q = synth.latent_inputs(w)
    say("noalloc: kv8 encode T=32768")
    codes, scales = kq.kv_encode_fp8(dev(x))
    out, lse = _both(kq.Cache.fp8(codes, scales), q, w.sm_scale, "kv8 T=32768 H=64")
    xh = o.kv8_decode(host(codes), host(scales))
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, w.sm_scale)
    check_attention(out, lse, ro, rl, "noalloc kv8 T=32768 H=64", twin=tw)
    # 2: smaller -- fewer rows and heads (fewer chunks of the same scratch)
    g = np.random.default_rng(31)
    x2 = (g.standard_normal((3001, 512)) * np.exp(g.standard_normal(512))).astype(np.float32)
    q2 = g.standard_normal((32, 512)).astype(np.float32)
    c2, s2 = kq.kv_encode_fp8(dev(x2))
    out2, lse2 = _both(kq.Cache.fp8(c2, s2), q2, 1 / np.sqrt(512), "kv8 T=3001 H=32")
    xh2 = o.kv8_decode(host(c2), host(s2))
    ro, rl, tw = reference(o.attention_decode, q2, xh2, xh2, 1 / np.sqrt(512))
    check_attention(out2, lse2, ro, rl, "noalloc kv8 T=3001 H=32", twin=tw)
    # 3: smaller still, another format through the same scratch: TQ4 (merge
    # and unrotate read the partials) and a q2k cache
    x3 = x2[:700]
    p3, r3 = kq.kv_encode_tq4(dev(x3), synth.ROT_SEED)
    out3, lse3 = _both(kq.Cache.tq4(p3, r3, synth.ROT_SEED), q2[:16], 1 / np.sqrt(512), "tq4 T=700 H=16")
    xh3 = o.tq4_decode(host(p3), host(r3), synth.ROT_SEED)
    ro, rl, tw = reference(o.attention_decode, q2[:16], xh3, xh3, 1 / np.sqrt(512))
    check_attention(out3, lse3, ro, rl, "noalloc tq4 T=700 H=16", twin=tw)
    K = (g.standard_normal((512, 2, 256)) * np.exp(1.5 * g.standard_normal((2, 256)))).astype(np.float32)
    V = (g.standard_normal((512, 2, 256)) * np.exp(1.5 * g.standard_normal((2, 256)))).astype(np.float32)
    enc = kq.kv_encode_q2k(dev(K), dev(V), 1.10, 8, 64)
    q4 = g.standard_normal((16, 256)).astype(np.float32)
    out4, lse4 = _both(kq.Cache.q2k(enc, 8, 64), q4, 1 / 16, "q2k T=512 16q/2kv")
    kc, ks, vb, ko, vo = o.q2k_encode(K, V, 1.10, 8, 64)
    Kd, Vd = o.q2k_decode(kc, ks, vb, ko, vo, 8, 64)
    ro, rl, tw = reference(o.attention_decode, q4, Kd, Vd, 1 / 16)
    check_attention(out4, lse4, ro, rl, "noalloc q2k T=512", twin=tw)


def test_noalloc_wide_tq4_decode_runs_per_head_group():
    """A TQ4 decode of 64 heads over a long cache plans all four head groups
    per workgroup, whose partials outgrow the scratch; without a workspace it
    runs per head group instead (another kernel, so the outputs are not
    bit-identical to the workspace call's: both must meet the bar)."""
    g = np.random.default_rng(47)
    T, d, H = 80000, 512, 64
    x = (g.standard_normal((T, d)) * np.exp(g.standard_normal(d))).astype(np.float32)
    q = g.standard_normal((H, d)).astype(np.float32)
    say(f"noalloc: tq4 encode T={T}")
    p, r = kq.kv_encode_tq4(dev(x), synth.ROT_SEED)
    cache = kq.Cache.tq4(p, r, synth.ROT_SEED)
    assert kq.attn_workspace_bytes(cache, H, 1) > (16 << 20)
    xh = o.tq4_decode(host(p), host(r), synth.ROT_SEED)
    ro, rl, tw = reference(o.attention_decode, q, xh, xh, 1 / np.sqrt(d))
    qd = dev(q)
    out_na = torch.full((H, d), -7.0, dtype=torch.float32, device=DEV)
    lse_na = torch.full((H,), -7.0, dtype=torch.float32, device=DEV)
    say(f"attn_decode_quant_noalloc tq4 T={T} H={H}")
    st = kq.lib.attn_decode_quant_noalloc(cache.ref, qd.data_ptr(), H, float(1 / np.sqrt(d)), out_na.data_ptr(),
                                          lse_na.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, kq.kvq_status_str(st)
    check_attention(host(out_na), host(lse_na), ro, rl, "noalloc tq4 T=80000 H=64", twin=tw)
    say(f"attn_decode_quant tq4 T={T} H={H}")
    out, lse = kq.attn_decode_quant(cache, qd, 1 / np.sqrt(d))
    check_attention(host(out), host(lse), ro, rl, "workspace tq4 T=80000 H=64", twin=tw)


def test_noalloc_refuses_requests_beyond_the_scratch():
    # the general f32 path at d = 1024 with 4096 heads needs 2 chunks x 4096
    # rows x 1026 floats = 33.6 MB of partials: refused, nothing written
    g = np.random.default_rng(32)
    x = g.standard_normal((4096, 1024)).astype(np.float32)
    codes, scales = kq.kv_encode_fp8(dev(x))
    cache = kq.Cache.fp8(codes, scales)
    assert kq.attn_workspace_bytes(cache, 4096, 1) > kq.NOALLOC_SCRATCH_BYTES
    q = dev(g.standard_normal((4096, 1024)).astype(np.float32))
    out = torch.full((4096, 1024), 3.0, dtype=torch.float32, device=DEV)
    say("attn_decode_quant_noalloc beyond the scratch")
    st = kq.lib.attn_decode_quant_noalloc(cache.ref, q.data_ptr(), 4096, 0.03, out.data_ptr(), None,
                                          torch.cuda.current_stream().cuda_stream)
    assert st == kq.KVQ_ERR_SCRATCH
    assert bool(torch.all(out == 3.0))
