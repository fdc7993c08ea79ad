"""Benchmark of the quantized-KV attention hot path on one MI355X.

Headline (the metric's configuration): KV8 decode, one query token, 64
absorbed heads, latent width 512 (key = value), T = 32768 cached rows ~
N(0,1) x lognormal(1) channel gains, fp8 e4m3 + f32 row scale.  One step is
one decode token through L = 64 cache instances ("layers"): per layer the new
row is encoded into its cache's last row and attention runs over all T rows,
one call (attn_decode_append_fp8: the decode launch encodes the row itself,
with the KV8 encoder's arithmetic and bytes).  64 x 16.9 MB = 1.08 GB of encoded KV per
step, so the caches cannot stay in the 256 MB last-level cache between
layers.  The step is captured once in a HIP graph and replayed.

    value = L * T * 516 B / step time   (GB/s of algorithmic KV bytes)

Also reported (same JSON line): the decode call's own duration from HIP
events on its stream (the roofline's `achieved`), the other hot-path rows
(tiny KV8 decode latency, TQ4 decode at T = 131072, q2k GQA decode at
T = 32768, KV8 chunked prefill S = 512 over T = 16384, KV8 decode at H = 8,
16, 32, multi-token, rope and top-k rows, the three encoders), each decode
row rotating >= 1 GiB of cache instances and each encoder row streaming
>= 1 GiB of input, and the CPU oracle timed per configuration at all host
threads and at one thread.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]

Profiler workloads and the summaries under profiles/ are in bench_profile.py.
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
F16_MFMA_PEAK_TFLOPS = 2500.0
SETTLE_MS = 150.0                # untimed back-to-back work before a timed region (clock ramp)
ROTATE_BYTES = 1 << 30          # every decode row rotates at least this much encoded cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------ inputs
def instances_for(bytes_each: float, floor: int = 1) -> int:
    """Cache instances to rotate so that their bytes reach ROTATE_BYTES."""
    return max(floor, int(np.ceil(ROTATE_BYTES / bytes_each)))


def device_rows(torch, n: int, d: int, seed: int, sigma: float = 1.0, dev="cuda:0"):
    """n rows ~ N(0,1) x per-channel lognormal(sigma) gains, drawn on the device."""
    g = torch.Generator(device=dev).manual_seed(seed)
    gains = torch.exp(sigma * torch.randn((d,), generator=g, device=dev))
    return torch.randn((n, d), generator=g, device=dev) * gains


def device_q2k_cells(torch, T: int, n_kv: int, d: int, seed: int, sigma: float, dev="cuda:0"):
    """K, V f32 [T, n_kv, d] ~ N(0,1) x per-(head, channel) lognormal(sigma) gains."""
    g = torch.Generator(device=dev).manual_seed(seed)
    gk = torch.exp(sigma * torch.randn((n_kv, d), generator=g, device=dev))
    gv = torch.exp(sigma * torch.randn((n_kv, d), generator=g, device=dev))
    K = torch.randn((T, n_kv, d), generator=g, device=dev) * gk
    V = torch.randn((T, n_kv, d), generator=g, device=dev) * gv
    return K, V


KV8_ENCODE_ROWS = 1 << 20       # 2 GiB of f32 input (512 wide)
TQ4_ENCODE_ROWS = 1 << 20
Q2K_ENCODE_CELLS = 1 << 18      # 2 x 512 MiB of f32 input (2 KV heads x 256)


# ------------------------------------------------------------ timing
class Timer:
    """HIP-event timing on the current stream."""

    def __init__(self, torch):
        self.t = torch

    def __call__(self, fn, reps):
        t = self.t
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        t.cuda.synchronize()
        return a.elapsed_time(b) / reps


def graph_timer(torch, fn, n=20, reps=5):
    """Device time per fn() call: n calls captured in one graph, best of reps
    replays (host launch overhead excluded); falls back to eager events."""
    fn()
    torch.cuda.synchronize()
    replay = capture(torch, lambda: [fn() for _ in range(n)])
    if replay is None:
        return Timer(torch)(fn, n)
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        replay()
        b.record()
        torch.cuda.synchronize()
        best = min(best, a.elapsed_time(b) / n)
    return best


def settle(torch, fn, ms):
    """Run fn() back to back for about `ms` of wall time: the GPU's clocks ramp
    up over the first tens of milliseconds of sustained work (a 2 ms prefill
    call measured 3.0, 2.4, 2.2, ... ms, steady at 1.8 ms after about 30 ms), so
    every timed region starts from the settled clock.  Untimed."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        fn()
        torch.cuda.synchronize()


def rotating_timer(torch, call, n_inst):
    """Device time per call(i) over instances i = 0 .. n_inst - 1, all of them
    captured in one graph (so a replay touches every instance once)."""
    k = [0]

    def one():
        call(k[0] % n_inst)
        k[0] += 1
    return graph_timer(torch, one, n=n_inst)


def capture(torch, fn):
    """Capture fn() into a graph; returns replay() or None if capture fails."""
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g.replay
    except Exception as e:  # pragma: no cover
        log(f"[bench] graph capture failed ({e}); timing eager launches")
        return None


_PHASES = []


def mark_phase(torch, name):
    """Start a named phase of the run (after the GPU has drained): the kernel
    summary assigns each traced dispatch to the phase whose window holds it."""
    torch.cuda.synchronize()
    _PHASES.append((name, time.clock_gettime_ns(time.CLOCK_BOOTTIME), time.monotonic_ns()))


# ------------------------------------------------------------ CPU oracle
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _timed(fn, seconds: float):
    """Seconds per fn() call: repeat until `seconds` have passed (at least once)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return el / reps, reps


def cpu_baseline(headline_seconds: float):
    """The oracle, as it stands, on a bounded sample of each configuration,
    at every BLAS thread the host gives numpy and again at one thread.

    The headline leg is one layer of the headline step (encode the new row,
    decode the cache rows to float64, float64 attention for 64 heads).  The
    other legs: the tiny KV8 decode call (encode its 256 rows + attention),
    the three encoders (rows or cells per second), the TQ4 decode over a
    prefix of its rows (scaled to T = 131072, the work being linear in T),
    the q2k decode call, and the KV8 prefill over its first tokens (scaled by
    the visible-row count to all 512 tokens, plus the encode of the 512 new
    rows and the decode of the cache to float64)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import kvq_oracle as o
    import synth

    blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    legs = {}

    # inputs (built once, not timed)
    w = synth.WORKLOADS["kv8_decode"]
    x, q = synth.latent_inputs(w)
    codes, scales = o.kv8_encode(x)

    def headline():
        c1, s1 = o.kv8_encode(x[-1:])
        codes[-1], scales[-1] = c1[0], s1[0]
        xh = o.kv8_decode(codes, scales)
        o.attention_decode(q, xh, xh, w.sm_scale)

    legs["kv8_decode_T32768_H64"] = (headline, headline_seconds, lambda s: (w.T * 516 / s / 1e9, "GB/s"),
                                     "single-layer decode steps (encode 1 row + f64 attention)")
    wt = synth.WORKLOADS["tiny_kv8"]
    xt, qt = synth.latent_inputs(wt)

    def tiny():
        c, s = o.kv8_encode(xt)
        xh = o.kv8_decode(c, s)
        o.attention_decode(qt, xh, xh, wt.sm_scale)
    legs["kv8_decode_tiny_H4_d64_T256"] = (tiny, 1.0, lambda s: (1.0 / s, "calls/s"),
                                           "calls (encode 256 rows + f64 attention)")
    xe = synth.encode_rows(2048)
    legs["kv8_encode"] = (lambda: o.kv8_encode(xe), 1.0, lambda s: (2048 / s, "rows/s"), "2048-row encodes")
    xe4 = synth.encode_rows(4096)
    legs["tq4_encode"] = (lambda: o.tq4_encode(xe4, synth.ROT_SEED), 1.0,
                          lambda s: (4096 / s, "rows/s"), "4096-row encodes")
    wq = synth.WORKLOADS["q2k_decode"]
    Ke, Ve, _ = synth.q2k_inputs(wq, T=4096)
    legs["q2k_encode"] = (lambda: o.q2k_encode(Ke, Ve, wq.k_gain, wq.n_sink, wq.n_window), 1.0,
                          lambda s: (4096 / s, "cells/s"), "4096-cell encodes (2 KV heads x 256)")
    w3 = synth.WORKLOADS["tq4_decode"]
    T3 = 8192
    x3, q3 = synth.latent_inputs(w3, T=T3)
    p3, r3 = o.tq4_encode(x3, synth.ROT_SEED)

    def tq4_part():
        xh = o.tq4_decode(p3, r3, synth.ROT_SEED)
        o.attention_decode(q3, xh, xh, w3.sm_scale)
    legs["tq4_decode_T131072_H64"] = (tq4_part, 1.0, lambda s: (1.0 / (s * w3.T / T3), "calls/s"),
                                      f"decodes of a {T3}-row prefix, scaled x{w3.T // T3} to T={w3.T}")
    K5, V5, q5 = synth.q2k_inputs(wq)
    enc5 = o.q2k_encode(K5, V5, wq.k_gain, wq.n_sink, wq.n_window)

    def q2k_call():
        Kh, Vh = o.q2k_decode(*enc5, wq.n_sink, wq.n_window)
        o.attention_decode(q5, Kh, Vh, wq.sm_scale)
    legs["q2k_decode_T32768"] = (q2k_call, 1.0, lambda s: (1.0 / s, "calls/s"), "full calls")
    w4 = synth.WORKLOADS["kv8_prefill"]
    x4, q4 = synth.latent_inputs(w4)
    c4, s4 = o.kv8_encode(x4[:w4.pos0])
    S_SAMPLE = 8
    rows_all = sum(w4.pos0 + s + 1 for s in range(w4.S))
    rows_part = sum(w4.pos0 + s + 1 for s in range(S_SAMPLE))
    x4n = x4[w4.pos0:]

    def prefill_fixed():
        cn, sn = o.kv8_encode(x4n)
        return o.kv8_decode(np.concatenate([c4, cn]), np.concatenate([s4, sn]))
    xh4 = prefill_fixed()
    legs["kv8_prefill_S512_T16384"] = (
        (prefill_fixed, lambda: o.attention_prefill(q4[:S_SAMPLE], xh4, xh4, w4.sm_scale, w4.pos0)),
        1.0, None,
        f"encode of the 512 new rows + cache decode, once, plus f64 attention of the first {S_SAMPLE} "
        f"tokens scaled by visible rows ({rows_part} of {rows_all})")

    rows = {}
    head = None
    for label, limit in (("all_threads", None), ("1_thread", 1)):
        with threadpool_limits(limits=limit):
            used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            for name, (fn, secs, conv, what) in legs.items():
                if name == "kv8_prefill_S512_T16384":
                    t_fixed, _ = _timed(fn[0], 0.0)
                    t_part, n = _timed(fn[1], secs)
                    val, unit = t_fixed + t_part * rows_all / rows_part, "s per call"
                else:
                    t, n = _timed(fn, secs)
                    val, unit = conv(t)
                rows.setdefault(name, {})[label] = {"value": float(f"{val:.4g}"), "unit": unit,
                                                    "threads": used, "reps": n, "sample": what}
                log(f"[bench] cpu oracle {name} ({label}): {val:.4g} {unit}")
                if name == "kv8_decode_T32768_H64" and head is None:
                    head = (val, used, n)
    val, used, n = head
    return {"value": round(val, 4), "unit": "GB/s", "cores": int(used), "kind": "oracle",
            "sample": f"{n} single-layer decode steps (encode 1 row + f64 attention, T=32768, H=64, "
                      f"d=512) in about {headline_seconds:.0f} s; numpy's BLAS ran {used} threads "
                      f"(elementwise numpy work is single-threaded)",
            "cpu_model": _cpu_model(), "cpus_available": int(avail), "blas_threads_default": int(blas),
            "configs": rows}


# ------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline only")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="seconds for the oracle's headline leg (per thread setting)")
    ap.add_argument("--phase-log", default=None,
                    help="write the host-clock windows of the run's phases (JSON) here")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              f"multi-GPU leg", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth
    import bench_profile

    dev = "cuda:0"

    # ------------------------------------------------------------ headline
    mark_phase(torch, "headline")
    w = synth.WORKLOADS["kv8_decode"]
    T, H, d, L = w.T, w.Hq, w.d, args.layers
    x, q = synth.latent_inputs(w)
    xd = torch.from_numpy(x).to(dev)
    qd = torch.from_numpy(q).to(dev)
    log(f"[bench] encoding {L} KV8 cache instances of T={T} d={d}")
    caches = []
    for _ in range(L):
        codes, scales = kq.kv_encode_fp8(xd)
        caches.append((codes, scales, kq.Cache.fp8(codes, scales)))
    ws = torch.empty((kq.attn_workspace_bytes(caches[0][2], H, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((H, d), dtype=torch.float32, device=dev)
    lse = torch.empty((H,), dtype=torch.float32, device=dev)
    new_row = xd[-1]

    def step():
        for _, _, cache in caches:
            kq.attn_decode_append_fp8(cache, new_row, qd, w.sm_scale, out=out, lse=lse, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    replay = None if args.no_graph else capture(torch, step)
    run = replay if replay is not None else step
    settle(torch, run, SETTLE_MS)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps x {L} layers ({'graph' if replay else 'eager'})")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / args.steps
    kv_bytes = T * kq.kvq_row_bytes("fp8", d)
    value = L * kv_bytes / (ms_step / 1e3) / 1e9

    # the step's call alone, HIP events on its stream, rotating the caches
    ev = []
    for _ in range(4):
        for _, _, cache in caches:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            kq.attn_decode_append_fp8(cache, new_row, qd, w.sm_scale, out=out, lse=lse, ws=ws)
            b.record()
            ev.append((a, b))
    torch.cuda.synchronize()
    decode_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    achieved = kv_bytes / (decode_us / 1e6) / 1e9
    tb = bench_profile.traffic_bytes_per_call("kv8_decode")
    traffic = None if tb is None else round(tb / (decode_us / 1e6) / 1e9, 2)
    log(f"[bench] step {ms_step:.3f} ms ({value:.0f} GB/s), decode call {decode_us:.1f} us "
        f"({achieved:.0f} GB/s)")

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
        "dtype": "f32 (f16 matrix-core operands, f32 accumulation)",
        "data": "synthetic",
        "config": {"workload": f"kv8_decode: 1 query token, H=64, d=512, T=32768 fp8 e4m3 rows; "
                               f"{L} cache instances per step (encode 1 row + decode each, one call)",
                   "T": T, "H": H, "d": d, "layers_per_step": L,
                   "launch": "hip graph" if replay else "eager",
                   "clock_settle_ms": SETTLE_MS},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     # measured HBM bytes per call over the same call duration
                     "traffic": traffic, "traffic_unit": "GB/s",
                     "traffic_bytes_per_call": None if tb is None else int(tb),
                     "algorithmic_bytes_per_call": int(kv_bytes),
                     "kernel": "attn_decode_append_fp8 (k_mla_mfma<KV8, append> + k_combine)",
                     "avg_us": round(decode_us, 2),
                     # the same call against the f16 matrix-core peak: 4*H*d flops per row
                     # (single-pass count; the kernel runs two passes for the f32 operand)
                     "mfma_tflops": round(4.0 * H * d * T / (decode_us / 1e6) / 1e12, 1),
                     "mfma_frac": round(4.0 * H * d * T / (decode_us / 1e6) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)},
    }
    del caches
    torch.cuda.empty_cache()

    if not args.no_extra:
        result["extra"] = extra_rows(torch, kq, synth)
    mark_phase(torch, "end")
    if args.phase_log:
        with open(args.phase_log, "w") as f:
            json.dump(_PHASES, f)

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle), headline leg {args.cpu_seconds} s per thread setting")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)

    print(json.dumps(result), flush=True)


def _row(us, nbytes):
    return {"us": round(us, 2), "GBps": round(nbytes / (us / 1e6) / 1e9, 1)}


def extra_rows(torch, kq, synth):
    """The other hot-path rows, each timed on its own workload."""
    dev = "cuda:0"
    res = {}
    timer = Timer(torch)

    # tiny KV8 decode (H = 4, d = 64, T = 256): a latency row
    mark_phase(torch, "tiny")
    w = synth.WORKLOADS["tiny_kv8"]
    x, q = synth.latent_inputs(w)
    xd, qd = torch.from_numpy(x).to(dev), torch.from_numpy(q).to(dev)
    c, s = kq.kv_encode_fp8(xd)
    cache = kq.Cache.fp8(c, s)
    ws = torch.empty((max(1, kq.attn_workspace_bytes(cache, w.Hq, 1)),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.Hq,), dtype=torch.float32, device=dev)
    us = graph_timer(torch, lambda: kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws),
                     n=64) * 1e3

    def enc_dec():
        kq.kv_encode_fp8(xd, c, s)
        kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws)
    us2 = graph_timer(torch, enc_dec, n=64) * 1e3
    res["kv8_decode_tiny_H4_d64_T256"] = {"us_per_call": round(us, 2), "calls_per_s": round(1e6 / us, 1),
                                          "us_encode_256_rows_and_decode": round(us2, 2)}
    del cache, c, s, xd, qd

    # TQ4 decode, T = 131072, rotating >= 1 GiB of caches
    mark_phase(torch, "tq4_decode")
    w = synth.WORKLOADS["tq4_decode"]
    x, q = synth.latent_inputs(w)
    xd = torch.from_numpy(x).to(dev)
    qd = torch.from_numpy(q).to(dev)
    b = w.T * kq.kvq_row_bytes("tq4", w.d)
    n_inst = instances_for(b)
    inst = []
    for _ in range(n_inst):
        p, r = kq.kv_encode_tq4(xd, synth.ROT_SEED)
        inst.append(kq.Cache.tq4(p, r, synth.ROT_SEED))
    del xd
    ws = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    ms = rotating_timer(torch, lambda i: kq.attn_decode_quant(inst[i], qd, w.sm_scale, out=out, ws=ws,
                                                              want_lse=False), n_inst)
    res["tq4_decode_T131072"] = {**_row(ms * 1e3, b), "instances": n_inst}
    del inst
    torch.cuda.empty_cache()

    # the encoders, each streaming >= 1 GiB of f32 input
    mark_phase(torch, "encoders")
    n, d = KV8_ENCODE_ROWS, 512
    xe = device_rows(torch, n, d, seed=1006)
    ce = torch.empty((n, d), dtype=torch.uint8, device=dev)
    se = torch.empty((n,), dtype=torch.float32, device=dev)
    kq.kv_encode_fp8(xe, ce, se)
    ms = timer(lambda: kq.kv_encode_fp8(xe, ce, se), 10)
    res["kv8_encode"] = {"rows": n, "rows_per_s": round(n / (ms / 1e3), 1),
                         "GBps": round(n * (4 * d + d + 4) / (ms / 1e3) / 1e9, 1)}
    del ce, se
    n = TQ4_ENCODE_ROWS
    pk = torch.empty((n, d // 2), dtype=torch.uint8, device=dev)
    rr = torch.empty((n,), dtype=torch.float32, device=dev)
    kq.kv_encode_tq4(xe[:n], synth.ROT_SEED, pk, rr)
    ms = timer(lambda: kq.kv_encode_tq4(xe[:n], synth.ROT_SEED, pk, rr), 10)
    res["tq4_encode"] = {"rows": n, "rows_per_s": round(n / (ms / 1e3), 1),
                         "GBps": round(n * (4 * d + d // 2 + 4) / (ms / 1e3) / 1e9, 1)}
    del xe, pk, rr
    torch.cuda.empty_cache()
    wq = synth.WORKLOADS["q2k_decode"]
    T = Q2K_ENCODE_CELLS
    Ke, Ve = device_q2k_cells(torch, T, wq.n_kv, wq.d, seed=1009, sigma=wq.sigma)
    enc = kq.kv_encode_q2k(Ke, Ve, wq.k_gain, wq.n_sink, wq.n_window)
    ms = timer(lambda: kq.kv_encode_q2k(Ke, Ve, wq.k_gain, wq.n_sink, wq.n_window, out=enc), 10)
    q2k_out = T * kq.kvq_row_bytes("q2k", wq.d, wq.n_kv)
    res["q2k_encode"] = {"cells": T, "cells_per_s": round(T / (ms / 1e3), 1),
                         "GBps": round((T * wq.n_kv * wq.d * 8 + q2k_out) / (ms / 1e3) / 1e9, 1)}
    del Ke, Ve, enc
    torch.cuda.empty_cache()

    # q2k GQA decode at T = 32768, rotating >= 1 GiB of caches
    mark_phase(torch, "q2k")
    w = wq
    K, V, q = synth.q2k_inputs(w)
    Kd, Vd, qd = (torch.from_numpy(a).to(dev) for a in (K, V, q))
    b = w.T * kq.kvq_row_bytes("q2k", w.d, w.n_kv)
    n_inst = instances_for(b)
    keep, inst = [], []
    for _ in range(n_inst):
        e = kq.kv_encode_q2k(Kd, Vd, w.k_gain, w.n_sink, w.n_window)
        keep.append(e)
        inst.append(kq.Cache.q2k(e, w.n_sink, w.n_window))
    ws = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    ms = rotating_timer(torch, lambda i: kq.attn_decode_quant(inst[i], qd, w.sm_scale, out=out, ws=ws,
                                                              want_lse=False), n_inst)
    res["q2k_decode_T32768"] = {**_row(ms * 1e3, b), "instances": n_inst}

    # q2k 4-token verify step (causal among the new tokens) over the same caches
    mark_phase(torch, "q2k_S4")
    qv = torch.randn((4, w.Hq, w.d), generator=torch.Generator(device=dev).manual_seed(47), device=dev)
    ws4 = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 4),), dtype=torch.uint8, device=dev)
    out4 = torch.empty((4, w.Hq, w.d), dtype=torch.float32, device=dev)
    ms = rotating_timer(torch, lambda i: kq.attn_prefill_quant(inst[i], qv, w.T - 4, w.sm_scale, out=out4,
                                                               ws=ws4, want_lse=False), n_inst)
    res["q2k_decode_S4_T32768"] = {**_row(ms * 1e3, b), "instances": n_inst}
    del keep, inst

    # q2k appends into a 32768-cell cache: one decode cell (its group
    # requantized from the cells present), and a 2048-cell prefill chunk that
    # starts mid-group
    mark_phase(torch, "q2k_append")
    buf = kq.q2k_alloc(w.T, w.n_kv, w.d, w.n_sink, w.n_window, 16)
    n0 = w.T - 2048 - 17
    kq.kv_append_q2k(Kd[:n0], Vd[:n0], 0, w.k_gain, w.n_sink, w.n_window, 16, buf)
    ms = graph_timer(torch, lambda: kq.kv_append_q2k(Kd[:n0 + 2048], Vd[:n0 + 2048], n0, w.k_gain,
                                                     w.n_sink, w.n_window, 16, buf), n=10)
    res["q2k_append_2048_cells"] = {"us": round(ms * 1e3, 1), "cells_per_s": round(2048 / (ms / 1e3), 1)}
    n1 = n0 + 2048
    ms = graph_timer(torch, lambda: kq.kv_append_q2k(Kd[:n1 + 1], Vd[:n1 + 1], n1, w.k_gain,
                                                     w.n_sink, w.n_window, 16, buf), n=20)
    res["q2k_append_1_cell"] = {"us": round(ms * 1e3, 1)}
    del buf, Kd, Vd
    torch.cuda.empty_cache()

    # KV8 chunked prefill: S = 512 new rows over T = 16384, 64 heads
    mark_phase(torch, "prefill")
    w = synth.WORKLOADS["kv8_prefill"]
    x, q = synth.latent_inputs(w)
    xd, qd = torch.from_numpy(x).to(dev), torch.from_numpy(q).to(dev)
    codes, scales = kq.kv_encode_fp8(xd)
    cache = kq.Cache.fp8(codes, scales)
    ws = torch.empty((kq.attn_workspace_bytes(cache, w.Hq, w.S),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.S, w.Hq, w.d), dtype=torch.float32, device=dev)

    def prefill():
        kq.kv_encode_fp8(xd[w.pos0:], codes[w.pos0:], scales[w.pos0:])
        kq.attn_prefill_quant(cache, qd, w.pos0, w.sm_scale, out=out, ws=ws, want_lse=False)
    settle(torch, prefill, SETTLE_MS)
    ms = timer(prefill, 5)
    rows = sum(w.pos0 + s + 1 for s in range(w.S))
    flops = 4.0 * w.Hq * w.d * rows                      # scores + context, one pass
    res["kv8_prefill_S512_T16384"] = {"ms": round(ms, 3), "TFLOPs": round(flops / (ms / 1e3) / 1e12, 2),
                                      "mfma_f16_frac": round(flops / (ms / 1e3) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)}
    del cache, codes, scales, xd, qd, out, ws
    torch.cuda.empty_cache()

    # KV8 decode at T = 32768 with fewer heads (where the decode turns from
    # matrix-core bound toward HBM bound), multi-token, rope and top-k rows,
    # each rotating >= 1 GiB of caches
    mark_phase(torch, "kv8_rows")
    w = synth.WORKLOADS["kv8_decode"]
    x, _ = synth.latent_inputs(w)
    xd = torch.from_numpy(x).to(dev)
    kv_bytes = w.T * kq.kvq_row_bytes("fp8", w.d)
    n_inst = instances_for(kv_bytes)
    inst = []
    for _ in range(n_inst):
        c, sc = kq.kv_encode_fp8(xd)
        inst.append(kq.Cache.fp8(c, sc))
    del xd
    # multi-token decode: S = 4 verify tokens (causal among them), 64 heads
    mark_phase(torch, "kv8_S4")
    qm = torch.randn((4, w.Hq, w.d), generator=torch.Generator(device=dev).manual_seed(44), device=dev)
    ws = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 4),), dtype=torch.uint8, device=dev)
    out = torch.empty((4, w.Hq, w.d), dtype=torch.float32, device=dev)
    ms = rotating_timer(torch, lambda i: kq.attn_prefill_quant(inst[i], qm, w.T - 4, w.sm_scale, out=out,
                                                               ws=ws, want_lse=False), n_inst)
    res["kv8_decode_S4_T32768"] = {**_row(ms * 1e3, kv_bytes), "instances": n_inst}
    for H in (8, 16, 32):
        mark_phase(torch, f"kv8_H{H}")
        qh = torch.randn((H, w.d), generator=torch.Generator(device=dev).manual_seed(H), device=dev)
        ws = torch.empty((kq.attn_workspace_bytes(inst[0], H, 1),), dtype=torch.uint8, device=dev)
        out = torch.empty((H, w.d), dtype=torch.float32, device=dev)
        ms = rotating_timer(torch, lambda i: kq.attn_decode_quant(inst[i], qh, w.sm_scale, out=out, ws=ws,
                                                                  want_lse=False), n_inst)
        res[f"kv8_decode_T32768_H{H}"] = {**_row(ms * 1e3, kv_bytes), "instances": n_inst}
    # the MLA key with its 64-wide rope part (GLM-5.2's 512 + 64 rows), 64 heads
    mark_phase(torch, "kv8_rope")
    gr = torch.Generator(device=dev).manual_seed(46)
    xr = torch.randn((w.T, 64), generator=gr, device=dev) * 3.0
    rope_inst = []
    for c in inst:
        rc, rs = kq.kv_encode_fp8(xr)
        rope_inst.append(kq.Cache.fp8(c.tensors[0], c.tensors[1], rope=(rc, rs)))
    qr = torch.randn((w.Hq, w.d + 64), generator=gr, device=dev)
    ws = torch.empty((kq.attn_workspace_bytes(rope_inst[0], w.Hq, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    ms = rotating_timer(torch, lambda i: kq.attn_decode_quant(rope_inst[i], qr, w.sm_scale, out=out, ws=ws,
                                                              want_lse=False), n_inst)
    r_bytes = w.T * (kq.kvq_row_bytes("fp8", w.d) + kq.kvq_row_bytes("fp8", 64))
    res["kv8_rope_decode_T32768"] = {**_row(ms * 1e3, r_bytes), "instances": n_inst}
    del rope_inst, xr

    # top-k sparse decode: 2048 listed rows of the 32768, 64 heads
    mark_phase(torch, "kv8_gather")
    idx = torch.from_numpy(synth.topk_rows(w.T, 2048, seed=1008)).to(dev)
    qg = torch.randn((w.Hq, w.d), generator=torch.Generator(device=dev).manual_seed(45), device=dev)
    ws = torch.empty((kq.attn_gather_workspace_bytes(inst[0], w.Hq, idx.numel()),), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    ms = rotating_timer(torch, lambda i: kq.attn_decode_gather(inst[i], idx, qg, w.sm_scale, out=out, ws=ws,
                                                               want_lse=False), n_inst)
    g_bytes = idx.numel() * (kq.kvq_row_bytes("fp8", w.d) + 4)   # rows + their list entries
    res["kv8_gather_top2048_T32768"] = {**_row(ms * 1e3, g_bytes), "instances": n_inst}
    del inst
    torch.cuda.empty_cache()

    mark_phase(torch, "device_copy")
    # a plain device copy (torch.neg, 1 GiB read + 1 GiB written): the HBM rate
    # an elementwise kernel reaches on this GPU, for context
    src = torch.empty((1 << 28,), dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    ms = timer(lambda: torch.neg(src, out=dst), 10)
    res["device_copy_GBps"] = round(2 * src.numel() * 4 / (ms / 1e3) / 1e9, 1)
    del src, dst
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
