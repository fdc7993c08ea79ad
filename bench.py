"""Benchmark of the quantized-KV attention hot path on one MI355X.

Headline (the metric's configuration): KV8 decode, one query token, 64
absorbed heads, latent width 512 (key = value), T = 32768 cached rows ~
N(0,1) x lognormal(1) channel gains, fp8 e4m3 + f32 row scale.  One step is
one decode token through L = 64 cache instances ("layers"): per layer the new
row is encoded into its cache (kv_encode_fp8, 1 row) and attention runs over
all T rows (attn_decode_quant).  64 x 16.9 MB = 1.08 GB of encoded KV per
step, so the caches cannot stay in the 256 MB last-level cache between
layers.  The step is captured once in a HIP graph and replayed.

    value = L * T * 516 B / step time   (GB/s of algorithmic KV bytes)

Also reported (same JSON line): the decode call's own duration from HIP
events on its stream (the roofline's `achieved`), the other hot-path rows
(TQ4 decode at T = 131072, q2k GQA decode at T = 32768, KV8 chunked prefill
S = 512 over T = 16384, and the three encoders' throughput), and the CPU
oracle timed on a bounded sample of the headline step.

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
F16_MFMA_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(x, q, sm_scale, T, seconds):
    """The oracle, as it stands, on one layer of the headline step: encode the
    new row, decode the cache rows to float64, float64 attention for 64 heads."""
    from oracle import kvq_oracle as o
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    codes, scales = o.kv8_encode(x)          # the cache (built once, not timed)
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
    return {"value": round(T * 516 / per / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{reps} single-layer decode steps (encode 1 row + f64 attention, T={T}, "
                      f"H=64, d=512) in {el:.1f} s, {per * 1e3:.1f} ms each"}


# ------------------------------------------------------------ HBM traffic
# roofline.traffic: HBM bytes per decode call from two rocprofv3 counter runs
# (FETCH_SIZE, then WRITE_SIZE) over `bench.py --traffic-probe`, each scaled
# by what the same counter reads for an elementwise kernel of known size
# (torch.neg over 256 MiB: 256 MiB read + 256 MiB written).  The summary file
# records a hash of the kernel sources it was taken on; bench.py reports the
# figure only while the sources still hash the same.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_kv8_decode.md")
TRAFFIC_SOURCES = ("attn_mla_mfma.hip", "attn_combine.hip", "kvq_internal.h")
PROBE_COPY_BYTES = 256 << 20
PROBE_CALLS = 8


def kernel_source_hash(sources=TRAFFIC_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "quantized_kv_cache_e4m3_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_probe():
    """The workload the counter runs profile: a known-size elementwise kernel,
    then PROBE_CALLS headline decode calls on one cache instance."""
    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth
    dev = "cuda:0"
    src = torch.ones(PROBE_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    w = synth.WORKLOADS["kv8_decode"]
    x, q = synth.latent_inputs(w)
    xd, qd = torch.from_numpy(x).to(dev), torch.from_numpy(q).to(dev)
    codes, scales = kq.kv_encode_fp8(xd)
    cache = kq.Cache.fp8(codes, scales)
    ws = torch.empty((kq.attn_workspace_bytes(cache, w.Hq, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    lse = torch.empty((w.Hq,), dtype=torch.float32, device=dev)
    for _ in range(PROBE_CALLS):
        # a cold cache each call: evict it from the last-level cache first
        torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws)
    torch.cuda.synchronize()
    print("traffic probe done", flush=True)


def mfma_probe():
    """The workload the matrix-core counter run profiles: the KV8 prefill
    (S=512, T=16384), the KV8 decode (T=32768, H=64) and the TQ4 decode
    (T=131072, H=64), a few calls each."""
    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth
    dev = "cuda:0"
    w = synth.WORKLOADS["kv8_prefill"]
    x, q = synth.latent_inputs(w)
    c, s = kq.kv_encode_fp8(torch.from_numpy(x).to(dev))
    cache, qd = kq.Cache.fp8(c, s), torch.from_numpy(q).to(dev)
    for _ in range(2):
        kq.attn_prefill_quant(cache, qd, w.pos0, w.sm_scale, want_lse=False)
    for name in ("kv8_decode", "tq4_decode"):
        w = synth.WORKLOADS[name]
        x, q = synth.latent_inputs(w)
        xd = torch.from_numpy(x).to(dev)
        if w.fmt == "tq4":
            p_, r_ = kq.kv_encode_tq4(xd, synth.ROT_SEED)
            cache = kq.Cache.tq4(p_, r_, synth.ROT_SEED)
        else:
            c, s = kq.kv_encode_fp8(xd)
            cache = kq.Cache.fp8(c, s)
        qd = torch.from_numpy(q).to(dev)
        for _ in range(4):
            kq.attn_decode_quant(cache, qd, w.sm_scale, want_lse=False)
    torch.cuda.synchronize()
    print("mfma probe done", flush=True)


def _counter_rows(path):
    import csv
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            rows[key] = rows.get(key, 0.0) + float(r["Counter_Value"])
    return rows


def traffic_summary(fetch_csv, write_csv, command):
    """Turn the two counter_collection.csv files into profiles/traffic_kv8_decode.md."""
    out = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        probe = [v for (i, k), v in rows.items() if "neg" in k.lower()]
        mla = [v for (i, k), v in sorted(rows.items()) if "k_mla_mfma" in k]
        comb = [v for (i, k), v in sorted(rows.items()) if "k_combine" in k]
        if not probe or not mla or not comb:
            raise SystemExit(f"{path}: missing probe ({len(probe)}), k_mla_mfma ({len(mla)}) "
                             f"or k_combine ({len(comb)}) dispatches")
        kib_probe = float(np.median(probe))
        scale = PROBE_COPY_BYTES / (kib_probe * 1024.0)
        out[name] = {"probe_kib": kib_probe, "scale": scale,
                     "mla_bytes": float(np.median(mla[1:] or mla)) * 1024.0 * scale,
                     "combine_bytes": float(np.median(comb[1:] or comb)) * 1024.0 * scale}
    total = sum(v["mla_bytes"] + v["combine_bytes"] for v in out.values())
    algo = 32768 * 516
    lines = [
        "# HBM traffic of one KV8 decode call (T=32768, H=64, d=512)",
        "",
        "Commands (run from the repository root, `$R` = its path):",
        "",
        "    " + command.replace("\n", "\n    "),
        "",
        "| counter | probe kernel (KiB) | scale to bytes | k_mla_mfma<KV8> (MB) | k_combine (MB) |",
        "|---|---|---|---|---|",
    ]
    for name, v in out.items():
        lines.append(f"| {name} | {v['probe_kib']:.0f} | {v['scale']:.4f} | "
                     f"{v['mla_bytes'] / 1e6:.3f} | {v['combine_bytes'] / 1e6:.3f} |")
    lines += [
        "",
        f"Probe: torch.neg over {PROBE_COPY_BYTES >> 20} MiB of f32 (that many bytes read and written); "
        f"each counter is scaled so that the probe reads exactly its known size.",
        f"Algorithmic bytes per call: {algo} (32768 rows x 516 B).",
        "",
        f"traffic_bytes_per_call: {total:.0f}",
        f"kernel_sources_sha: {kernel_source_hash()}",
    ]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_util_prefill_decode.md")
MFMA_SOURCES = ("attn_mla_prefill.hip", "attn_mla_mfma.hip", "kvq_internal.h")
SIMDS, CLOCK_HZ, XCDS, F16_PEAK = 1024, 2.4e9, 8, 2.5e15


def mfma_summary(csv_path, command):
    """Turn the matrix-core counter run of --mfma-probe into a summary: per
    kernel, the f16 MFMA work the hardware counted against the algorithmic
    flops, and the fraction of SIMD cycles the matrix cores were busy."""
    import csv
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            k = _short_kernel(r["Kernel_Name"])
            d = per.setdefault(k, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    hd = 4 * 64 * 512
    pf = synth_prefill_flops()
    cases = [("k_mla_prefill_kv8", "KV8 prefill, S=512, T=16384, H=64", pf),
             ("k_mla_mfma<1, false, false>", "KV8 decode, T=32768, H=64", hd * 32768),
             ("k_mla_mfma<2, false, false>", "TQ4 decode, T=131072, H=64", hd * 131072)]
    lines = [
        "# Matrix-core utilisation of the attention kernels (rocprofv3 counters)",
        "",
        "Commands (run from the repository root, `$R` = its path):",
        "",
        "    " + command.replace("\n", "\n    "),
        "",
        "| kernel | workload | dispatches | kernel time (us, median) | MFMA f16 flops counted | "
        "algorithmic flops | counted / algorithmic | MFMA rate (TFLOP/s) | of the 2.5 PFLOP/s f16 peak | "
        "MFMA busy / SIMD cycles at 2.4 GHz | MFMA busy / GPU-active cycles |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for k, what, algo in cases:
        ds = list(per.get(k, {}).values())
        if not ds:
            raise SystemExit(f"{csv_path}: no {k} dispatches")
        med = lambda key: float(np.median([d[key] for d in ds]))
        ns, mops = med("ns"), med("SQ_INSTS_VALU_MFMA_MOPS_F16")
        busy, gui = med("SQ_VALU_MFMA_BUSY_CYCLES"), med("GRBM_GUI_ACTIVE")
        flops = mops * 512.0
        rate = flops / (ns * 1e-9)
        lines.append(f"| `{k}` | {what} | {len(ds)} | {ns / 1e3:.1f} | {flops:.4e} | {algo:.4e} | "
                     f"{flops / algo:.3f} | {rate / 1e12:.0f} | {100 * rate / F16_PEAK:.1f} % | "
                     f"{100 * busy / (ns * 1e-9 * CLOCK_HZ * SIMDS):.1f} % | "
                     f"{100 * busy / (gui / XCDS * SIMDS):.1f} % |")
    lines += [
        "",
        "Counters: `SQ_INSTS_VALU_MFMA_MOPS_F16` counts f16 matrix work in units of 512 flops; "
        "`SQ_VALU_MFMA_BUSY_CYCLES` sums the cycles the matrix cores were busy over all "
        f"{SIMDS} SIMDs; `GRBM_GUI_ACTIVE` sums the GPU-active cycles over the {XCDS} XCDs.",
        "The last column is rocprofv3's MfmaUtil (busy / (per-XCD active cycles x SIMDs)); for a kernel of a few "
        "microseconds the active window includes the counter set-up around the dispatch, so the column before it "
        "(busy cycles over the kernel's own duration at the 2.4 GHz peak clock) is the figure to use there.",
        "Algorithmic flops: 4 H d per visible (query, row) pair (score and value products); the prefill is causal "
        "with pos0 = T - S.",
        "",
        f"kernel_sources_sha: {kernel_source_hash(MFMA_SOURCES)}",
    ]
    with open(MFMA_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def synth_prefill_flops() -> float:
    S, T, H, d = 512, 16384, 64, 512
    pos0 = T - S
    return 4.0 * H * d * (S * pos0 + S * (S + 1) / 2)


KERNEL_SUMMARY_FILE = os.path.join(ROOT, "profiles", "kernels_bench_default.md")


def _short_kernel(name):
    import re
    m = re.search(r"(k_[a-z0-9_]+)(<[^>]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return "torch: " + name.split("(")[0].split("::")[-1][:40]


# what each kernel is in each phase of the default run: (phase, kernel, grid)
# or (phase, kernel) for every launch shape of that kernel in the phase
KERNEL_ROLES = {
    ("headline", "k_mla_mfma<1, false, false>", 131072): "KV8 decode, T=32768, H=64 (256 workgroups: 64 chunks x 4 head groups)",
    ("headline", "k_combine"): "chunk merge of the KV8 decode (64 rows x 8 dim slices, one wave each)",
    ("headline", "k_encode_fp8_vec<1>", 256): "KV8 encode of the 1 appended row per layer (timed step)",
    ("headline", "k_encode_fp8_vec<1>", 2097152): "KV8 encode of 32768 rows (cache set-up)",
    ("tq4_decode", "k_mla_mfma<2, false, false>"): "TQ4 decode, T=131072, H=64 (256 workgroups)",
    ("tq4_decode", "k_combine_unrotate512"): "TQ4 chunk merge + inverse rotation (one workgroup per query row)",
    ("tq4_decode", "k_encode_tq4_512"): "TQ4 encode of 131072 rows (set-up and encoder row)",
    ("kv8_encode", "k_encode_fp8_vec<1>"): "KV8 encode of 2^20 rows (encoder throughput row)",
    ("q2k", "k_q2k_mfma"): "q2k decode, T=32768, 2 KV heads x 8 query heads (256 workgroups)",
    ("q2k", "k_combine"): "chunk merge of the q2k decode (16 rows x 4 dim slices)",
    ("q2k", "k_encode_q2k"): "q2k encode of 32768 cells: K groups, V blocks and the fp16 overlay in one launch",
    ("q2k_S4", "k_q2k_mfma"): "q2k 4-token verify step, T=32768 (4 tokens x 2 KV heads x 32 slices)",
    ("q2k_S4", "k_combine"): "chunk merge of the q2k verify step",
    ("q2k_append", "k_append_q2k", 1280): "q2k append of 1 decode cell in one launch: its group requantized, V blocks, ring slot",
    ("q2k_append", "k_append_q2k", 1114624): "q2k append of 2048 cells from mid-group in one launch (65 groups requantized)",
    ("q2k_append", "k_append_q2k", 16702720): "q2k append of the 30703-cell prefix (set-up)",
    ("q2k_append", "k_append_q2k"): "q2k append in one launch: touched groups requantized, V blocks, ring overlay",
    ("prefill", "k_mla_prefill_kv8"): "KV8 chunked prefill, S=512, T=16384 (128 token groups x 4 head groups)",
    ("prefill", "k_encode_fp8_vec<1>", 32768): "KV8 encode of the 512 new prefill rows",
    ("prefill", "k_encode_fp8_vec<1>", 1048576): "KV8 encode of 16384 rows (prefill cache set-up)",
    ("kv8_small", "k_encode_fp8_vec<1>"): "KV8 encode of 32768 rows (cache set-up)",
    ("kv8_S4", "k_mla_mfma<1, false, false>"): "KV8 4-token decode (verify step), T=32768, H=64",
    ("kv8_S4", "k_combine"): "chunk merge of the 4-token decode (256 query rows)",
    ("kv8_H16", "k_mla_mfma<1, false, false>"): "KV8 decode, T=32768, H=16 (256 chunks x 1 head group)",
    ("kv8_H16", "k_combine"): "chunk merge, 16 query rows, 256 chunks",
    ("kv8_H32", "k_mla_mfma<1, false, false>"): "KV8 decode, T=32768, H=32 (128 chunks x 2 head groups)",
    ("kv8_H32", "k_combine"): "chunk merge, 32 query rows, 128 chunks",
    ("kv8_gather", "k_mla_mfma<1, false, true>"): "KV8 top-k gather decode, 2048 listed rows of 32768, H=64",
    ("kv8_gather", "k_combine"): "chunk merge of the gather decode (16 chunks)",
    ("kv8_rope", "k_mla_mfma<1, true, false>"): "KV8 decode with the 64-wide rope key part, T=32768, H=64",
    ("kv8_rope", "k_combine"): "chunk merge of the rope decode",
    ("kv8_rope", "k_encode_fp8_vec<1>"): "KV8 encode of the 32768 rope rows (set-up)",
    ("device_copy", "torch: neg_kernel_cuda"): "plain device copy, 1 GiB read + 1 GiB written (HBM reference rate)",
}

_PHASES = []


def mark_phase(torch, name):
    """Start a named phase of the run (after the GPU has drained): the kernel
    summary assigns each traced dispatch to the phase whose window holds it."""
    torch.cuda.synchronize()
    _PHASES.append((name, time.clock_gettime_ns(time.CLOCK_BOOTTIME), time.monotonic_ns()))


def _assign_phases(disp, phase_log):
    """disp: [(start_ns, end_ns, key)].  Returns phase names per dispatch, using
    whichever host clock (boot time or monotonic) the trace's timestamps follow:
    the one that places more dispatches inside a phase window."""
    with open(phase_log) as f:
        ph = json.load(f)
    best = None
    for ci in (1, 2):
        names = []
        for st, en, _ in disp:
            nm = "unassigned"
            for j in range(len(ph) - 1):
                if ph[j][ci] <= st and en <= ph[j + 1][ci]:
                    nm = ph[j][0]
                    break
            names.append(nm)
        hit = sum(n != "unassigned" for n in names)
        if best is None or hit > best[0]:
            best = (hit, names, "CLOCK_BOOTTIME" if ci == 1 else "CLOCK_MONOTONIC")
    return best[1], best[2]


def kernel_summary(trace_csv, command, phase_log=None):
    """Per (phase, kernel, launch shape) durations from a rocprofv3 kernel_trace.csv."""
    import csv
    import collections
    disp = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            key = (_short_kernel(r["Kernel_Name"]), grid, int(r["Workgroup_Size_X"]), int(r["LDS_Block_Size"]))
            disp.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), key))
    clock = None
    if phase_log:
        names, clock = _assign_phases(disp, phase_log)
    else:
        names = ["-"] * len(disp)
    agg = collections.defaultdict(list)
    for (st, en, key), nm in zip(disp, names):
        agg[(nm,) + key].append((en - st) / 1e3)
    lines = [
        "# Kernel durations of the default `bench.py` run",
        "",
        "Command (run from the repository root, `$R` = its path):",
        "",
        "    " + command,
        "",
        "Durations are rocprofv3 kernel-trace start/end per dispatch (no launch gaps), grouped by",
        "the bench phase the dispatch ran in, kernel and launch shape (grid = total threads)."
        + (f"  Phases from the run's phase log ({clock} windows)." if clock else ""),
        "",
        "| phase | kernel | grid | block | LDS (B) | calls | mean us | median us | min us | max us | what it is |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    order = [p[0] for p in json.load(open(phase_log))] if phase_log else []
    rows = sorted(agg.items(), key=lambda kv: (order.index(kv[0][0]) if kv[0][0] in order else len(order),
                                               -sum(kv[1])))
    for (ph, name, grid, block, lds), v in rows:
        if name.startswith("torch:") and sum(v) < 1000.0:
            continue
        role = KERNEL_ROLES.get((ph, name, grid), KERNEL_ROLES.get((ph, name), ""))
        if not role and name.startswith("torch:"):
            role = "benchmark input generation"
        lines.append(f"| {ph} | `{name}` | {grid} | {block} | {lds} | {len(v)} | {np.mean(v):.2f} | "
                     f"{np.median(v):.2f} | {np.min(v):.2f} | {np.max(v):.2f} | {role} |")
    with open(KERNEL_SUMMARY_FILE, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_bytes_per_call():
    """Measured HBM bytes per decode call, or None when not measured on these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    vals = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith(("|", " ", "#")))
    if vals.get("kernel_sources_sha", "").strip() != kernel_source_hash():
        return None
    try:
        return float(vals["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline only")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only the workload the HBM-traffic counter runs profile")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("COUNTER_CSV", "COMMAND"),
                    help="write the matrix-core utilisation summary from a --mfma-probe counter run")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="run only the workload the matrix-core counter run profiles")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "COMMAND"),
                    help="write profiles/traffic_kv8_decode.md from the two counter runs")
    ap.add_argument("--kernel-summary", nargs="+", metavar="ARG",
                    help="TRACE_CSV COMMAND [PHASE_LOG]: write profiles/kernels_bench_default.md "
                         "from a rocprofv3 kernel trace")
    ap.add_argument("--phase-log", default=None,
                    help="write the host-clock windows of the run's phases (JSON) here")
    args = ap.parse_args()
    if args.kernel_summary:
        if len(args.kernel_summary) not in (2, 3):
            ap.error("--kernel-summary TRACE_CSV COMMAND [PHASE_LOG]")
        kernel_summary(*args.kernel_summary)
        return
    if args.mfma_summary:
        mfma_summary(*args.mfma_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path has no "
              f"multi-GPU leg", file=sys.stderr)
        sys.exit(2)

    if args.traffic_probe:
        traffic_probe()
        return
    if args.mfma_probe:
        mfma_probe()
        return

    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth

    dev = "cuda:0"
    timer = Timer(torch)

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
    new_row = xd[-1:]

    def step():
        for codes, scales, cache in caches:
            kq.kv_encode_fp8(new_row, codes[-1:], scales[-1:])
            kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    replay = None if args.no_graph else capture(torch, step)
    run = replay if replay is not None else step
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

    # the decode call alone, HIP events on its stream, rotating the caches
    ev = []
    for _ in range(4):
        for codes, scales, cache in caches:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws)
            b.record()
            ev.append((a, b))
    torch.cuda.synchronize()
    decode_us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    achieved = kv_bytes / (decode_us / 1e6) / 1e9
    tb = traffic_bytes_per_call()
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
                               f"{L} cache instances per step (encode 1 row + decode each)",
                   "T": T, "H": H, "d": d, "layers_per_step": L,
                   "launch": "hip graph" if replay else "eager"},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "attn_decode_quant (k_mla_mfma<KV8> + k_combine)",
                     "avg_us": round(decode_us, 2),
                     # the same call against the f16 matrix-core peak: 4*H*d flops per row
                     # (single-pass count; the kernel runs two passes for the f32 operand)
                     "mfma_tflops": round(4.0 * H * d * T / (decode_us / 1e6) / 1e12, 1),
                     "mfma_frac": round(4.0 * H * d * T / (decode_us / 1e6) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)},
    }
    del caches
    torch.cuda.empty_cache()

    if not args.no_extra:
        result["extra"] = extra_rows(torch, kq, synth, timer)
    mark_phase(torch, "end")
    if args.phase_log:
        with open(args.phase_log, "w") as f:
            json.dump(_PHASES, f)

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) for ~{args.cpu_seconds} s")
        result["cpu_baseline"] = cpu_baseline(x, q, w.sm_scale, T, args.cpu_seconds)

    print(json.dumps(result), flush=True)


def extra_rows(torch, kq, synth, timer):
    """The other hot-path rows, each timed on its own workload."""
    dev = "cuda:0"
    res = {}

    # TQ4 decode, T = 131072 (8 cache instances rotated: 272 MB)
    mark_phase(torch, "tq4_decode")
    w = synth.WORKLOADS["tq4_decode"]
    x, q = synth.latent_inputs(w)
    xd = torch.from_numpy(x).to(dev)
    qd = torch.from_numpy(q).to(dev)
    inst = []
    for _ in range(8):
        p, r = kq.kv_encode_tq4(xd, synth.ROT_SEED)
        inst.append(kq.Cache.tq4(p, r, synth.ROT_SEED))
    ws = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    k = [0]

    def tq4_call():
        kq.attn_decode_quant(inst[k[0] % 8], qd, w.sm_scale, out=out, ws=ws, want_lse=False)
        k[0] += 1
    ms = graph_timer(torch, tq4_call, n=16)
    b = w.T * kq.kvq_row_bytes("tq4", w.d)
    res["tq4_decode_T131072"] = {"us": round(ms * 1e3, 1), "GBps": round(b / (ms / 1e3) / 1e9, 1)}

    # TQ4 encoder on those rows (rows/s)
    pk = torch.empty((w.T, w.d // 2), dtype=torch.uint8, device=dev)
    rr = torch.empty((w.T,), dtype=torch.float32, device=dev)
    ms = timer(lambda: kq.kv_encode_tq4(xd, synth.ROT_SEED, pk, rr), 10)
    res["tq4_encode_rows_per_s"] = round(w.T / (ms / 1e3), 1)
    del inst, xd, pk, rr
    torch.cuda.empty_cache()

    # KV8 encoder, 2^20 rows x 512 (2 GiB of f32 input)
    mark_phase(torch, "kv8_encode")
    n, d = 1 << 20, 512
    g = torch.Generator(device=dev).manual_seed(1006)
    xe = torch.randn((n, d), generator=g, device=dev) * torch.exp(torch.randn((d,), generator=g, device=dev))
    ce = torch.empty((n, d), dtype=torch.uint8, device=dev)
    se = torch.empty((n,), dtype=torch.float32, device=dev)
    kq.kv_encode_fp8(xe, ce, se)
    ms = timer(lambda: kq.kv_encode_fp8(xe, ce, se), 10)
    res["kv8_encode_rows_per_s"] = round(n / (ms / 1e3), 1)
    res["kv8_encode_GBps"] = round(n * (4 * d + d + 4) / (ms / 1e3) / 1e9, 1)
    del xe, ce, se
    torch.cuda.empty_cache()

    mark_phase(torch, "q2k")
    # q2k: encode (cells/s) and GQA decode at T = 32768 (20 cache instances
    # rotated: 294 MB, more than the last-level cache)
    w = synth.WORKLOADS["q2k_decode"]
    K, V, q = synth.q2k_inputs(w)
    Kd, Vd, qd = (torch.from_numpy(a).to(dev) for a in (K, V, q))
    enc = kq.kv_encode_q2k(Kd, Vd, w.k_gain, w.n_sink, w.n_window)
    ms = timer(lambda: kq.kv_encode_q2k(Kd, Vd, w.k_gain, w.n_sink, w.n_window, out=enc), 10)
    res["q2k_encode_cells_per_s"] = round(w.T / (ms / 1e3), 1)
    inst = [kq.Cache.q2k(enc, w.n_sink, w.n_window)]
    keep = [enc]
    for _ in range(19):
        e = kq.kv_encode_q2k(Kd, Vd, w.k_gain, w.n_sink, w.n_window)
        keep.append(e)
        inst.append(kq.Cache.q2k(e, w.n_sink, w.n_window))
    ws = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 1),), dtype=torch.uint8, device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    k = [0]

    def q2k_call():
        kq.attn_decode_quant(inst[k[0] % 20], qd, w.sm_scale, out=out, ws=ws, want_lse=False)
        k[0] += 1
    ms = graph_timer(torch, q2k_call, n=20)
    b = w.T * kq.kvq_row_bytes("q2k", w.d, w.n_kv)
    res["q2k_decode_T32768"] = {"us": round(ms * 1e3, 1), "GBps": round(b / (ms / 1e3) / 1e9, 1)}

    # q2k appends into a 32768-cell cache: one decode cell (its group
    # requantized from the cells present), and a 2048-cell prefill chunk that
    # starts mid-group
    mark_phase(torch, "q2k_append")
    buf = kq.q2k_alloc(w.T, w.n_kv, w.d, w.n_sink, w.n_window, 16)
    kq.kv_append_q2k(Kd[:w.T - 2048 - 17], Vd[:w.T - 2048 - 17], 0, w.k_gain, w.n_sink, w.n_window, 16, buf)
    n0 = w.T - 2048 - 17
    ms = graph_timer(torch, lambda: kq.kv_append_q2k(Kd[:n0 + 2048], Vd[:n0 + 2048], n0, w.k_gain,
                                                     w.n_sink, w.n_window, 16, buf), n=10)
    res["q2k_append_2048_cells"] = {"us": round(ms * 1e3, 1), "cells_per_s": round(2048 / (ms / 1e3), 1)}
    n1 = n0 + 2048
    ms = graph_timer(torch, lambda: kq.kv_append_q2k(Kd[:n1 + 1], Vd[:n1 + 1], n1, w.k_gain,
                                                     w.n_sink, w.n_window, 16, buf), n=20)
    res["q2k_append_1_cell"] = {"us": round(ms * 1e3, 1)}
    del buf
    # q2k 4-token verify step (causal among the new tokens) over the same caches
    qv = torch.randn((4, w.Hq, w.d), generator=torch.Generator(device=dev).manual_seed(47), device=dev)
    ws4 = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 4),), dtype=torch.uint8, device=dev)
    out4 = torch.empty((4, w.Hq, w.d), dtype=torch.float32, device=dev)
    k[0] = 0
    mark_phase(torch, "q2k_S4")

    def q2k_verify():
        kq.attn_prefill_quant(inst[k[0] % 20], qv, w.T - 4, w.sm_scale, out=out4, ws=ws4, want_lse=False)
        k[0] += 1
    ms = graph_timer(torch, q2k_verify, n=20)
    res["q2k_decode_S4_T32768"] = {"us": round(ms * 1e3, 1), "GBps": round(b / (ms / 1e3) / 1e9, 1)}
    del enc, keep, inst, Kd, Vd
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
    prefill()
    ms = timer(prefill, 3)
    rows = sum(w.pos0 + s + 1 for s in range(w.S))
    flops = 4.0 * w.Hq * w.d * rows                      # scores + context, one pass
    res["kv8_prefill_S512_T16384"] = {"ms": round(ms, 3), "TFLOPs": round(flops / (ms / 1e3) / 1e12, 2),
                                      "mfma_f16_frac": round(flops / (ms / 1e3) / 1e12 / F16_MFMA_PEAK_TFLOPS, 4)}
    del cache, codes, scales, xd, qd, out, ws
    torch.cuda.empty_cache()

    # KV8 decode at T = 32768 with fewer heads: where the decode turns from
    # matrix-core bound (64 heads, 254 flop per KV byte) toward HBM bound
    mark_phase(torch, "kv8_small")
    w = synth.WORKLOADS["kv8_decode"]
    x, _ = synth.latent_inputs(w)
    xd = torch.from_numpy(x).to(dev)
    inst = []
    for _ in range(16):                                  # 16 x 16.9 MB rotated, beyond the MALL
        c, sc = kq.kv_encode_fp8(xd)
        inst.append(kq.Cache.fp8(c, sc))
    del xd
    kv_bytes = w.T * kq.kvq_row_bytes("fp8", w.d)
    # multi-token decode: S = 4 verify tokens (causal among them), 64 heads
    qm = torch.randn((4, w.Hq, w.d), generator=torch.Generator(device=dev).manual_seed(44), device=dev)
    ws = torch.empty((kq.attn_workspace_bytes(inst[0], w.Hq, 4),), dtype=torch.uint8, device=dev)
    out = torch.empty((4, w.Hq, w.d), dtype=torch.float32, device=dev)
    k = [0]
    mark_phase(torch, "kv8_S4")

    def mtp():
        kq.attn_prefill_quant(inst[k[0] % 16], qm, w.T - 4, w.sm_scale, out=out, ws=ws, want_lse=False)
        k[0] += 1
    ms = graph_timer(torch, mtp, n=16)
    res["kv8_decode_S4_T32768"] = {"us": round(ms * 1e3, 1), "GBps": round(kv_bytes / (ms / 1e3) / 1e9, 1)}
    for H in (16, 32):
        qh = torch.randn((H, w.d), generator=torch.Generator(device=dev).manual_seed(H), device=dev)
        ws = torch.empty((kq.attn_workspace_bytes(inst[0], H, 1),), dtype=torch.uint8, device=dev)
        out = torch.empty((H, w.d), dtype=torch.float32, device=dev)
        k = [0]
        mark_phase(torch, f"kv8_H{H}")

        def call():
            kq.attn_decode_quant(inst[k[0] % 16], qh, w.sm_scale, out=out, ws=ws, want_lse=False)
            k[0] += 1
        ms = graph_timer(torch, call, n=16)
        res[f"kv8_decode_T32768_H{H}"] = {"us": round(ms * 1e3, 1), "GBps": round(kv_bytes / (ms / 1e3) / 1e9, 1)}
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
    k = [0]

    def rope_call():
        kq.attn_decode_quant(rope_inst[k[0] % 16], qr, w.sm_scale, out=out, ws=ws, want_lse=False)
        k[0] += 1
    ms = graph_timer(torch, rope_call, n=16)
    r_bytes = w.T * (kq.kvq_row_bytes("fp8", w.d) + kq.kvq_row_bytes("fp8", 64))
    res["kv8_rope_decode_T32768"] = {"us": round(ms * 1e3, 1), "GBps": round(r_bytes / (ms / 1e3) / 1e9, 1)}
    del rope_inst, xr

    # top-k sparse decode: 2048 listed rows of the 32768, 64 heads
    mark_phase(torch, "kv8_gather")
    idx = torch.from_numpy(synth.topk_rows(w.T, 2048, seed=1008)).to(dev)
    qg = torch.randn((w.Hq, w.d), generator=torch.Generator(device=dev).manual_seed(45), device=dev)
    ws = torch.empty((kq.attn_gather_workspace_bytes(inst[0], w.Hq, idx.numel()),), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
    k = [0]

    def gather():
        kq.attn_decode_gather(inst[k[0] % 16], idx, qg, w.sm_scale, out=out, ws=ws, want_lse=False)
        k[0] += 1
    ms = graph_timer(torch, gather, n=16)
    g_bytes = idx.numel() * (kq.kvq_row_bytes("fp8", w.d) + 4)   # rows + their list entries
    res["kv8_gather_top2048_T32768"] = {"us": round(ms * 1e3, 1), "GBps": round(g_bytes / (ms / 1e3) / 1e9, 1)}
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
