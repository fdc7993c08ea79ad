"""Profiler workloads for bench.py's figures, and the summaries under profiles/.

Each summary is written from a rocprofv3 run of one of the probe workloads
below and records the command that made it.

  HBM traffic (FETCH_SIZE, then WRITE_SIZE, each a counter run of its own):
    rocprofv3 --pmc FETCH_SIZE -d <dir> -o run -- python -u bench_profile.py probe <workload>
    python bench_profile.py traffic <workload> FETCH_CSV WRITE_CSV "<commands>"
  Matrix-core utilisation:
    rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE ... \
        -- python -u bench_profile.py mfma-probe
    python bench_profile.py mfma COUNTER_CSV "<commands>"
  Kernel durations of the default bench run:
    rocprofv3 --kernel-trace --stats ... -- python -u bench.py --phase-log PHASES.json
    python bench_profile.py kernels TRACE_CSV "<command>" PHASES.json

Traffic counters are scaled by what the same counter reads for a plain
elementwise kernel of known size (torch.neg over 256 MiB of f32: that many
bytes read and as many written), run first in the same process.  A summary
records a hash of the kernel sources it was taken on; bench.py reports the
traffic figure only while the sources still hash the same.
"""
from __future__ import annotations

import csv
import collections
import hashlib
import json
import os
import re
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
PROFILES = os.path.join(ROOT, "profiles")
PROBE_COPY_BYTES = 256 << 20
PROBE_CALLS = 6


def kernel_source_hash(sources) -> str:
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "quantized_kv_cache_e4m3_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_kernel(name):
    m = re.search(r"(k_[a-z0-9_]+)(<[^>]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return "torch: " + name.split("(")[0].split("::")[-1][:40]


# ------------------------------------------------------------ traffic workloads
def _q2k_row_bytes():
    import quantized_kv_cache_e4m3_amd as kq
    return kq.kvq_row_bytes("q2k", 256, 2)


# name -> title, kernels (short-name prefix, label), sources hashed, algorithmic
# bytes per call (a function: some need the library's row-size helper), text
TRAFFIC = {
    "kv8_decode": dict(
        title="one KV8 decode step call (attn_decode_append_fp8: the new row encoded in the decode "
              "launch, T=32768, H=64, d=512)",
        kernels=[("k_mla_mfma<1", "k_mla_mfma<KV8, append>"), ("k_combine", "k_combine")],
        sources=("attn_mla_mfma.hip", "attn_combine.hip", "kvq_internal.h"),
        algo=lambda: 32768 * 516 + 2048,
        algo_text="32768 rows x 516 B (fp8 row + f32 scale; the new one written, the others read) + the "
                  "2048 B f32 new row"),
    "tq4_decode": dict(
        title="one TQ4 decode call (T=131072, H=64, d=512)",
        kernels=[("k_prep_query", "k_prep_query<TQ4>"), ("k_mla_tiles<2", "k_mla_tiles<TQ4, decode>"),
                 ("k_combine", "k_combine"), ("k_unrotate", "k_unrotate")],
        sources=("attn_mla_prefill.hip", "attn_mla_mfma.hip", "attn_combine.hip", "kvq_internal.h"),
        algo=lambda: 131072 * 260, algo_text="131072 rows x 260 B (256 B of nibbles + f32 radius)"),
    "q2k_decode": dict(
        title="one q2k GQA decode call (T=32768, 2 KV heads x 256, 16 query heads)",
        kernels=[("k_q2k_mfma", "k_q2k_mfma"), ("k_combine_q2k", "k_combine_q2k")],
        sources=("attn_q2k_mfma.hip", "kvq_internal.h"),
        algo=lambda: int(32768 * _q2k_row_bytes()),
        algo_text="32768 cells x the q2k bytes per cell of 2 KV heads (K codes + K scales + V blocks + overlay)"),
    "kv8_encode": dict(
        title="one KV8 encode of 2^20 rows x 512",
        kernels=[("k_encode_fp8", "k_encode_fp8")],
        sources=("encode.hip", "kvq_internal.h"),
        algo=lambda: (1 << 20) * (2048 + 516), algo_text="2^20 rows x (2048 B f32 in + 516 B out)"),
    "tq4_encode": dict(
        title="one TQ4 encode of 2^20 rows x 512",
        kernels=[("k_encode_tq4", "k_encode_tq4")],
        sources=("encode.hip", "kvq_internal.h"),
        algo=lambda: (1 << 20) * (2048 + 260), algo_text="2^20 rows x (2048 B f32 in + 260 B out)"),
    "q2k_encode": dict(
        title="one q2k encode of 2^18 cells (2 KV heads x 256)",
        kernels=[("k_encode_q2k", "k_encode_q2k")],
        sources=("encode.hip", "kvq_internal.h"),
        algo=lambda: int((1 << 18) * (2 * 256 * 8 + _q2k_row_bytes())),
        algo_text="2^18 cells x (4096 B of f32 K and V in + the q2k bytes per cell out)"),
}


def traffic_file(name):
    return os.path.join(PROFILES, f"traffic_{name}.md")


def probe(name):
    """The workload a traffic counter run profiles: the known-size elementwise
    kernel, then PROBE_CALLS calls of the workload (decodes: each on caches
    evicted from the last-level cache first)."""
    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth
    import bench
    dev = "cuda:0"
    src = torch.ones(PROBE_COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst

    def evict():
        torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)

    if name in ("kv8_decode", "tq4_decode"):
        w = synth.WORKLOADS[name]
        x, q = synth.latent_inputs(w)
        xd, qd = torch.from_numpy(x).to(dev), torch.from_numpy(q).to(dev)
        if w.fmt == "tq4":
            p, r = kq.kv_encode_tq4(xd, synth.ROT_SEED)
            cache = kq.Cache.tq4(p, r, synth.ROT_SEED)
        else:
            c, s = kq.kv_encode_fp8(xd)
            cache = kq.Cache.fp8(c, s)
        ws = torch.empty((kq.attn_workspace_bytes(cache, w.Hq, 1),), dtype=torch.uint8, device=dev)
        out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
        lse = torch.empty((w.Hq,), dtype=torch.float32, device=dev)
        for _ in range(PROBE_CALLS):
            evict()
            if w.fmt == "tq4":
                kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, lse=lse, ws=ws)
            else:       # the decode step as the bench times it: the new row encoded in the launch
                kq.attn_decode_append_fp8(cache, xd[-1], qd, w.sm_scale, out=out, lse=lse, ws=ws)
    elif name == "q2k_decode":
        w = synth.WORKLOADS[name]
        K, V, q = synth.q2k_inputs(w)
        Kd, Vd, qd = (torch.from_numpy(a).to(dev) for a in (K, V, q))
        enc = kq.kv_encode_q2k(Kd, Vd, w.k_gain, w.n_sink, w.n_window)
        cache = kq.Cache.q2k(enc, w.n_sink, w.n_window)
        ws = torch.empty((kq.attn_workspace_bytes(cache, w.Hq, 1),), dtype=torch.uint8, device=dev)
        out = torch.empty((w.Hq, w.d), dtype=torch.float32, device=dev)
        for _ in range(PROBE_CALLS):
            evict()
            kq.attn_decode_quant(cache, qd, w.sm_scale, out=out, ws=ws, want_lse=False)
    elif name in ("kv8_encode", "tq4_encode"):
        n, d = 1 << 20, 512
        xe = bench.device_rows(torch, n, d, seed=1006)
        if name == "kv8_encode":
            ce = torch.empty((n, d), dtype=torch.uint8, device=dev)
            se = torch.empty((n,), dtype=torch.float32, device=dev)
            for _ in range(PROBE_CALLS):
                kq.kv_encode_fp8(xe, ce, se)
        else:
            pk = torch.empty((n, d // 2), dtype=torch.uint8, device=dev)
            rr = torch.empty((n,), dtype=torch.float32, device=dev)
            for _ in range(PROBE_CALLS):
                kq.kv_encode_tq4(xe, synth.ROT_SEED, pk, rr)
    elif name == "q2k_encode":
        w = synth.WORKLOADS["q2k_decode"]
        Ke, Ve = bench.device_q2k_cells(torch, 1 << 18, w.n_kv, w.d, seed=1009, sigma=w.sigma)
        enc = kq.kv_encode_q2k(Ke, Ve, w.k_gain, w.n_sink, w.n_window)
        for _ in range(PROBE_CALLS):
            kq.kv_encode_q2k(Ke, Ve, w.k_gain, w.n_sink, w.n_window, out=enc)
    else:
        raise SystemExit(f"unknown traffic workload {name!r}; one of {sorted(TRAFFIC)}")
    torch.cuda.synchronize()
    print(f"traffic probe {name} done", flush=True)


def _counter_rows(path):
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            rows[key] = rows.get(key, 0.0) + float(r["Counter_Value"])
    return rows


def traffic_summary(name, fetch_csv, write_csv, command):
    """Turn the two counter_collection.csv files into profiles/traffic_<name>.md."""
    spec = TRAFFIC[name]
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path)
        probe_kib = [v for (i, k), v in rows.items() if "neg" in k.lower()]
        if not probe_kib:
            raise SystemExit(f"{path}: no probe (torch.neg) dispatch")
        kib = float(np.median(probe_kib))
        scale = PROBE_COPY_BYTES / (kib * 1024.0)
        ks = {}
        for prefix, label in spec["kernels"]:
            vals = [v for (i, k), v in sorted(rows.items()) if short_kernel(k).startswith(prefix)
                    and not any(short_kernel(k).startswith(p) for p, _ in spec["kernels"]
                                if p != prefix and p.startswith(prefix))]
            if not vals:
                raise SystemExit(f"{path}: no {label} dispatches")
            ks[label] = (float(np.median(vals[1:] or vals)) * 1024.0 * scale, len(vals))
        per[counter] = (kib, scale, ks)
    algo = spec["algo"]()
    total = sum(b for _, _, ks in per.values() for b, _ in ks.values())
    labels = [label for _, label in spec["kernels"]]
    lines = [
        f"# HBM traffic of {spec['title']}",
        "",
        "Commands (run from the repository root, `$R` = its path):",
        "",
        "    " + command.replace("\n", "\n    "),
        "",
        "| counter | probe kernel (KiB) | scale to bytes | " + " | ".join(f"{l} (MB)" for l in labels) + " |",
        "|---|---|---|" + "---|" * len(labels),
    ]
    for counter, (kib, scale, ks) in per.items():
        lines.append(f"| {counter} | {kib:.0f} | {scale:.4f} | "
                     + " | ".join(f"{ks[l][0] / 1e6:.3f}" for l in labels) + " |")
    lines += [
        "",
        f"Probe: torch.neg over {PROBE_COPY_BYTES >> 20} MiB of f32 (that many bytes read and written); "
        f"each counter is scaled so that the probe reads exactly its known size.  Per kernel: the median "
        f"over the workload's dispatches after the first ({per['FETCH_SIZE'][2][labels[0]][1]} dispatches).",
        f"Algorithmic bytes per call: {algo} ({spec['algo_text']}).",
        f"Measured / algorithmic: {total / algo:.3f}",
        "",
        f"traffic_bytes_per_call: {total:.0f}",
        f"kernel_sources_sha: {kernel_source_hash(spec['sources'])}",
    ]
    with open(traffic_file(name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic_bytes_per_call(name):
    """Measured HBM bytes per call of workload `name`, or None when not
    measured on the current kernel sources."""
    try:
        with open(traffic_file(name)) as f:
            text = f.read()
    except OSError:
        return None
    vals = dict(l.split(": ", 1) for l in text.splitlines() if ": " in l and not l.startswith(("|", " ", "#")))
    if vals.get("kernel_sources_sha", "").strip() != kernel_source_hash(TRAFFIC[name]["sources"]):
        return None
    try:
        return float(vals["traffic_bytes_per_call"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------ matrix cores
MFMA_FILE = os.path.join(PROFILES, "mfma_util_attention.md")
MFMA_SOURCES = ("attn_mla_prefill.hip", "attn_mla_mfma.hip", "attn_q2k_mfma.hip", "kvq_internal.h")
SIMDS, CLOCK_HZ, XCDS, F16_PEAK = 1024, 2.4e9, 8, 2.5e15


def mfma_probe():
    """The workload the matrix-core counter run profiles: the KV8 prefill
    (S=512, T=16384), the KV8 decode (T=32768, H=64), the TQ4 decode
    (T=131072, H=64) and the q2k decode (T=32768).  Each runs enough calls
    that the median dispatch is one at the settled clock (the GPU's clocks
    ramp up over the first tens of milliseconds of sustained work)."""
    import torch
    import quantized_kv_cache_e4m3_amd as kq
    import synth
    dev = "cuda:0"
    w = synth.WORKLOADS["kv8_prefill"]
    x, q = synth.latent_inputs(w)
    c, s = kq.kv_encode_fp8(torch.from_numpy(x).to(dev))
    cache, qd = kq.Cache.fp8(c, s), torch.from_numpy(q).to(dev)
    for _ in range(24):
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
        for _ in range(32):
            kq.attn_decode_quant(cache, qd, w.sm_scale, want_lse=False)
    w = synth.WORKLOADS["q2k_decode"]
    K, V, q = synth.q2k_inputs(w)
    Kd, Vd, qd = (torch.from_numpy(a).to(dev) for a in (K, V, q))
    cache = kq.Cache.q2k(kq.kv_encode_q2k(Kd, Vd, w.k_gain, w.n_sink, w.n_window), w.n_sink, w.n_window)
    for _ in range(32):
        kq.attn_decode_quant(cache, qd, w.sm_scale, want_lse=False)
    torch.cuda.synchronize()
    print("mfma probe done", flush=True)


def prefill_flops() -> float:
    S, T, H, d = 512, 16384, 64, 512
    pos0 = T - S
    return 4.0 * H * d * (S * pos0 + S * (S + 1) / 2)


def mfma_summary(csv_path, command):
    """Per kernel: the f16 MFMA work the hardware counted against the
    algorithmic flops, and the fraction of SIMD cycles the matrix cores were
    busy."""
    per = {}
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            k = short_kernel(r["Kernel_Name"])
            d = per.setdefault(k, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    hd = 4 * 64 * 512
    cases = [("k_mla_tiles<1, 0>", "KV8 prefill, S=512, T=16384, H=64", prefill_flops()),
             ("k_mla_mfma<1, false, false, false>", "KV8 decode, T=32768, H=64", hd * 32768),
             ("k_mla_tiles<2, 1>", "TQ4 decode, T=131072, H=64", hd * 131072),
             ("k_q2k_mfma", "q2k decode, T=32768, 16 query heads x 256", 4 * 16 * 256 * 32768)]
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
        ds = [v for kk, dd in per.items() if kk.startswith(k) for v in dd.values()]
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


# ------------------------------------------------------------ kernel durations
KERNEL_SUMMARY_FILE = os.path.join(PROFILES, "kernels_bench_default.md")

# what each kernel is in each phase of the default run: (phase, kernel, grid)
# or (phase, kernel) for every launch shape of that kernel in the phase
KERNEL_ROLES = {
    ("headline", "k_mla_mfma<1, false, false, true>", 131072): "KV8 decode step, T=32768, H=64: the appended row encoded by the decode launch itself (256 workgroups: 64 chunks x 4 head groups)",
    ("headline", "k_combine"): "chunk merge of the KV8 decode (64 rows x 8 dim slices, two waves of 32 chunks each)",
    ("headline", "k_encode_fp8_vec<1>", 2097152): "KV8 encode of 32768 rows (cache set-up)",
    ("tiny", "k_attn_split<1, 1>"): "tiny KV8 decode, H=4, d=64, T=256 (general f32 path, 16 chunks of one tile)",
    ("tiny", "k_combine"): "chunk merge of the tiny decode",
    ("tiny", "k_encode_fp8_vec<1>"): "KV8 encode of the tiny cache's 256 rows",
    ("tq4_decode", "k_prep_query"): "TQ4 decode: query rotated and split into f16 halves once (one wave per head)",
    ("tq4_decode", "k_mla_tiles<2, 1>"): "TQ4 decode, T=131072, H=64: one workgroup per 512-row chunk takes all 64 heads (256 workgroups)",
    ("tq4_decode", "k_combine"): "chunk merge of the TQ4 decode (256 chunks; 64 rows x 8 dim slices)",
    ("tq4_decode", "k_unrotate512"): "TQ4 inverse rotation of the merged context, once per head",
    ("tq4_decode", "k_encode_tq4_512"): "TQ4 encode of 131072 rows (cache set-up)",
    ("encoders", "k_encode_fp8_vec<1>"): "KV8 encode of 2^20 rows (encoder row)",
    ("encoders", "k_encode_tq4_512"): "TQ4 encode of 2^20 rows (encoder row)",
    ("encoders", "k_encode_q2k"): "q2k encode of 2^18 cells: K groups, V blocks and the fp16 overlay in one launch",
    ("q2k", "k_q2k_mfma"): "q2k decode of the bulk cells, and of the 256 window cells on the 8 waves per KV head that have no bulk group, T=32768, 2 KV heads x 8 query heads (128 slices x 2 KV heads)",
    ("q2k", "k_combine_q2k<1>"): "q2k combine: the 8 sink cells attended in f32, merged with the 128 bulk partials (16 rows x 4 slices; one 64-cell round, every load before the first wait)",
    ("q2k", "k_encode_q2k"): "q2k encode of 32768 cells (cache set-up)",
    ("q2k_S4", "k_q2k_mfma"): "q2k 4-token verify step, T=32768",
    ("q2k_S4", "k_combine_q2k<5>"): "q2k combine of the verify step (the whole overlay in five 64-cell rounds + bulk partials)",
    ("q2k_append", "k_append_q2k", 1280): "q2k append of 1 decode cell in one launch: its group requantized, V blocks, ring slot",
    ("q2k_append", "k_append_q2k"): "q2k append in one launch: touched groups requantized, V blocks, ring overlay",
    ("prefill", "k_mla_tiles<1, 0>"): "KV8 chunked prefill, S=512, T=16384 (128 token groups x 4 head groups, one wave per SIMD)",
    ("prefill", "k_encode_fp8_vec<1>", 32768): "KV8 encode of the 512 new prefill rows",
    ("prefill", "k_encode_fp8_vec<1>", 1048576): "KV8 encode of 16384 rows (prefill cache set-up)",
    ("kv8_rows", "k_encode_fp8_vec<1>"): "KV8 encode of 32768 rows (cache set-up)",
    ("kv8_S4", "k_mla_mfma<1, false, false, false>"): "KV8 4-token decode (verify step), T=32768, H=64",
    ("kv8_S4", "k_combine"): "chunk merge of the 4-token decode (256 query rows)",
    ("kv8_H8", "k_mla_mfma<1, false, false, false>"): "KV8 decode, T=32768, H=8 (one head group, padded to 16)",
    ("kv8_H8", "k_combine"): "chunk merge, 8 query rows",
    ("kv8_H16", "k_mla_mfma<1, false, false, false>"): "KV8 decode, T=32768, H=16 (1 head group)",
    ("kv8_H16", "k_combine"): "chunk merge, 16 query rows",
    ("kv8_H32", "k_mla_mfma<1, false, false, false>"): "KV8 decode, T=32768, H=32 (2 head groups)",
    ("kv8_H32", "k_combine"): "chunk merge, 32 query rows",
    ("kv8_gather", "k_mla_mfma<1, false, true, false>"): "KV8 top-k gather decode, 2048 listed rows of 32768, H=64",
    ("kv8_gather", "k_combine"): "chunk merge of the gather decode",
    ("kv8_rope", "k_mla_mfma<1, true, false, false>"): "KV8 decode with the 64-wide rope key part, T=32768, H=64",
    ("kv8_rope", "k_combine"): "chunk merge of the rope decode",
    ("kv8_rope", "k_encode_fp8_vec<1>"): "KV8 encode of the 32768 rope rows (set-up)",
    ("device_copy", "torch: neg_kernel_cuda"): "plain device copy, 1 GiB read + 1 GiB written (HBM reference rate)",
}


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
    disp = []
    with open(trace_csv) as f:
        for r in csv.DictReader(f):
            grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            key = (short_kernel(r["Kernel_Name"]), grid, int(r["Workgroup_Size_X"]), int(r["LDS_Block_Size"]))
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


def main(argv):
    usage = ("bench_profile.py probe WORKLOAD | traffic WORKLOAD FETCH_CSV WRITE_CSV COMMAND | "
             "mfma-probe | mfma COUNTER_CSV COMMAND | kernels TRACE_CSV COMMAND [PHASE_LOG]")
    if not argv:
        raise SystemExit(usage)
    cmd, rest = argv[0], argv[1:]
    if cmd == "probe" and len(rest) == 1:
        probe(rest[0])
    elif cmd == "traffic" and len(rest) == 4:
        traffic_summary(*rest)
    elif cmd == "mfma-probe" and not rest:
        mfma_probe()
    elif cmd == "mfma" and len(rest) == 2:
        mfma_summary(*rest)
    elif cmd == "kernels" and len(rest) in (2, 3):
        kernel_summary(*rest)
    else:
        raise SystemExit(usage)


if __name__ == "__main__":
    main(sys.argv[1:])
