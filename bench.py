"""Benchmark: decode attention over an fp8 (KV8) MLA-latent cache on one GPU.

Workload (the metric's configuration): one query token, 64 absorbed heads,
latent width 512 (key = value), T = 32768 cached rows ~ N(0,1) x lognormal(1)
channel gains, encoded as fp8 e4m3 + f32 row scale.  One step is one decode
token through L = 64 cache instances ("layers"): for each layer, the new row
is encoded into its cache (kv_encode_fp8, 1 row) and attention runs over all
T rows (attn_decode_quant).  64 x 16.9 MB = 1.08 GB of encoded KV per step,
so the caches cannot sit in the 256 MB last-level cache between layers.

value = algorithmic KV bytes read per step (L * T * 516 B) / step time, GB/s.
Also reported: the decode call's own average duration from HIP events on the
stream it runs on (the roofline's `achieved`), encoder throughput in rows/s on
2^20 rows, and the CPU oracle timed on a bounded sample of the same step.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(x, q, sm_scale, T, seconds):
    """The oracle, as it stands, on one layer of the step: encode the new row,
    decode the cache rows to float64 and run float64 attention for 64 heads."""
    from oracle import kvq_oracle as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    codes, scales = o.kv8_encode(x)          # the cache (not timed: built once)
    reps, t0 = 0, time.perf_counter()
    while True:
        c1, s1 = o.kv8_encode(x[-1:])
        codes[-1], scales[-1] = c1[0], s1[0]
        xh = o.kv8_decode(codes, scales)
        o.attention_decode(q, xh, xh, sm_scale)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds and reps >= 2:
            break
    per = el / reps
    return {"value": T * 516 / per / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{reps} single-layer decode steps (encode 1 row + f64 attention, T={T}, "
                      f"H=64, d=512) in {el:.1f} s, {per * 1e3:.1f} ms each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-encode", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              f"multi-GPU leg in this build", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth

    dev = "cuda:0"
    w = synth.WORKLOADS["kv8_decode"]
    T, H, d, L = w.T, w.Hq, w.d, args.layers
    x, q = synth.latent_inputs(w)
    xd = torch.from_numpy(x).to(dev)
    qd = torch.from_numpy(q).to(dev)
    log(f"[bench] encoding {L} cache instances of T={T} d={d}")
    caches = []
    for _ in range(L):
        codes, scales = kq.kv_encode_fp8(xd)
        caches.append((codes, scales, kq.Cache.fp8(codes, scales)))
    ws = torch.empty((kq.attn_workspace_bytes(caches[0][2], H, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((H, d), dtype=torch.float32, device=dev)
    lse = torch.empty((H,), dtype=torch.float32, device=dev)
    new_row = xd[-1:]

    def step(events=None):
        for li, (codes, scales, cache) in enumerate(caches):
            kq.kv_encode_fp8(new_row, codes[-1:], scales[-1:])
            if events is not None:
                events[li][0].record()
            kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws)
            if events is not None:
                events[li][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(L)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps x {L} layers")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(ev[k])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / args.steps
    durs = [a.elapsed_time(b) for row in ev for (a, b) in row]
    decode_ms = float(np.mean(durs))
    kv_bytes = T * kq.kvq_row_bytes("fp8", d)
    value = L * kv_bytes / (ms_step / 1e3) / 1e9
    achieved = kv_bytes / (decode_ms / 1e3) / 1e9
    log(f"[bench] step {ms_step:.3f} ms, decode call {decode_ms * 1e3:.1f} us, "
        f"{achieved:.0f} GB/s per call")

    result = {
        "metric": "decode-attn KV GB/s (% of HBM peak) at T=32k/128k; encode rows/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kv8_decode: 1 query token, H=64, d=512, T=32768 fp8 e4m3 rows, "
                               f"{L} cache instances per step (encode 1 row + decode each)",
                   "T": T, "H": H, "d": d, "layers_per_step": L},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "attn_decode_quant (split + combine kernels)",
                     "avg_us": round(decode_ms * 1e3, 2)},
    }

    if not args.no_encode:
        n = 1 << 20
        g = torch.Generator(device=dev).manual_seed(1006)
        gains = torch.exp(torch.randn((d,), generator=g, device=dev))
        xe = torch.randn((n, d), generator=g, device=dev) * gains
        ce = torch.empty((n, d), dtype=torch.uint8, device=dev)
        se = torch.empty((n,), dtype=torch.float32, device=dev)
        for _ in range(2):
            kq.kv_encode_fp8(xe, ce, se)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        a.record()
        for _ in range(reps):
            kq.kv_encode_fp8(xe, ce, se)
        b.record()
        torch.cuda.synchronize()
        enc_ms = a.elapsed_time(b) / reps
        result["encode_rows_per_s"] = round(n / (enc_ms / 1e3), 1)
        result["encode_GBps"] = round(n * (d * 4 + d + 4) / (enc_ms / 1e3) / 1e9, 2)
        del xe, ce, se

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) for ~{args.cpu_seconds} s")
        result["cpu_baseline"] = cpu_baseline(x, q, w.sm_scale, T, args.cpu_seconds)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
