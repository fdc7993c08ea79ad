"""Seeded synthetic inputs shared by the oracle tests and the GPU path.

This module draws random arrays and nothing else: it holds none of the
method's arithmetic (no encoding, rotation, codebook or attention step).  All
arrays are float32 host arrays from numpy's PCG64 generator.

Workloads (shapes from the pages: the MLA latent row of width 512 shared by
64 absorbed query heads in colibri #399 / #553, and Strata #2318's 2 KV heads
x 256 dims with 8 query heads per KV head; the channel structure is a
lognormal per-channel gain, standing in for the channel spread that page
measures on real K and V):

  tiny_kv8     T=256,    H=4,  d=64   rows ~ N(0,1)                 seed 1001
  kv8_decode   T=32768,  H=64, d=512  rows ~ N(0,1) * exp(N(0,1))   seed 1002
  tq4_decode   T=131072, H=64, d=512  as kv8_decode                 seed 1003
  kv8_prefill  S=512 new rows, T=16384, H=64, d=512 (pos0 = 15872)  seed 1004
  q2k_decode   T=32768, 2 KV heads x 256, 16 query heads,
               K, V ~ N(0,1) * exp(1.5 N(0,1)) per (head, channel)   seed 1005
  encode_rows  2^20 rows of width 512 as kv8_decode                 seed 1006
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

ROT_SEED = 0x5EED000000000003


@dataclass
class Workload:
    name: str
    fmt: str            # "fp8" | "tq4" | "q2k"
    T: int              # cached rows (cells)
    Hq: int             # query heads
    d: int              # row width (per KV head for q2k)
    n_kv: int = 1
    S: int = 1          # query tokens (prefill: new rows)
    pos0: int = 0       # prefill: absolute position of query 0
    sigma: float = 1.0  # lognormal gain sigma (0: no gains)
    seed: int = 0
    k_gain: float = 1.10
    n_sink: int = 8
    n_window: int = 256

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "tiny_kv8": Workload("tiny_kv8", "fp8", T=256, Hq=4, d=64, sigma=0.0, seed=1001),
    "kv8_decode": Workload("kv8_decode", "fp8", T=32768, Hq=64, d=512, sigma=1.0, seed=1002),
    "tq4_decode": Workload("tq4_decode", "tq4", T=131072, Hq=64, d=512, sigma=1.0, seed=1003),
    "kv8_prefill": Workload("kv8_prefill", "fp8", T=16384, Hq=64, d=512, S=512, pos0=16384 - 512,
                            sigma=1.0, seed=1004),
    "q2k_decode": Workload("q2k_decode", "q2k", T=32768, Hq=16, d=256, n_kv=2, sigma=1.5, seed=1005),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def gained_rows(g: np.random.Generator, n: int, d: int, sigma: float) -> np.ndarray:
    """n rows of width d: N(0,1) times one lognormal(sigma) gain per channel."""
    gains = np.exp(sigma * g.standard_normal(d)).astype(np.float32) if sigma > 0 else None
    x = g.standard_normal((n, d), dtype=np.float32)
    if gains is not None:
        x *= gains[None, :]
    return x


def latent_inputs(w: Workload, T: int | None = None, Hq: int | None = None):
    """(rows f32 [T, d], q f32 [Hq, d] or [S, Hq, d]) for a KV8 / TQ4 workload.
    Smaller T / Hq give a prefix-shaped case drawn from the same recipe."""
    T = w.T if T is None else T
    Hq = w.Hq if Hq is None else Hq
    g = rng(w.seed)
    x = gained_rows(g, T, w.d, w.sigma)
    if w.S > 1:
        q = g.standard_normal((w.S, Hq, w.d), dtype=np.float32)
    else:
        q = g.standard_normal((Hq, w.d), dtype=np.float32)
    return x, q


def q2k_inputs(w: Workload, T: int | None = None):
    """(K f32 [T, n_kv, d], V f32 [T, n_kv, d], q f32 [Hq, d]) for q2k."""
    T = w.T if T is None else T
    g = rng(w.seed)
    gk = np.exp(w.sigma * g.standard_normal((w.n_kv, w.d))).astype(np.float32)
    gv = np.exp(w.sigma * g.standard_normal((w.n_kv, w.d))).astype(np.float32)
    K = g.standard_normal((T, w.n_kv, w.d), dtype=np.float32) * gk[None]
    V = g.standard_normal((T, w.n_kv, w.d), dtype=np.float32) * gv[None]
    q = g.standard_normal((w.Hq, w.d), dtype=np.float32)
    return K, V, q


def encode_rows(n: int = 1 << 20, d: int = 512, seed: int = 1006, sigma: float = 1.0) -> np.ndarray:
    """The encoder-throughput row set (2^20 x 512 f32 = 2 GiB by default)."""
    return gained_rows(rng(seed), n, d, sigma)


def edge_rows(d: int, seed: int = 77) -> np.ndarray:
    """Edge-case rows: zeros, a single spike, a constant row, +-0 mixes, tiny
    and huge magnitudes, subnormals, and values at e4m3 rounding midpoints of
    the row scale."""
    g = rng(seed)
    rows = []
    rows.append(np.zeros(d, np.float32))
    r = np.zeros(d, np.float32); r[d // 3] = 5.0; rows.append(r)
    rows.append(np.full(d, -2.5, np.float32))
    r = np.zeros(d, np.float32); r[::2] = -0.0; r[1] = 1.0; rows.append(r)
    rows.append((g.standard_normal(d) * 1e-30).astype(np.float32))
    rows.append((g.standard_normal(d) * 1e30).astype(np.float32))
    rows.append((g.standard_normal(d) * 1e-39).astype(np.float32))   # subnormal f32
    # values k/16 of 448 on a unit-scale row: many land on e4m3 rounding ties
    r = (np.arange(d, dtype=np.float32) % 64 - 32) / np.float32(16.0) * np.float32(14.0)
    r[0] = 448.0
    rows.append(r.astype(np.float32))
    r = g.standard_normal(d).astype(np.float32); r[5] = 1e4; rows.append(r)
    return np.stack(rows).astype(np.float32)


def tiny_amax_rows(d: int, n: int = 64, seed: int = 78, lo: float = 3e-43, hi: float = 1.3e-42) -> np.ndarray:
    """Rows whose largest magnitude lies in [lo, hi] (f32 subnormals): n rows
    with amax swept evenly over the range, +amax at element 0 and -amax at
    element 1 (d >= 2), the rest uniform in (-amax, amax)."""
    g = rng(seed)
    amax = np.linspace(lo, hi, n).astype(np.float32)
    u = g.uniform(-1.0, 1.0, (n, d)).astype(np.float32)
    rows = (u * amax[:, None]).astype(np.float32)
    rows[:, 0] = amax
    if d >= 2:
        rows[:, 1] = -amax
    return rows


def topk_rows(T: int, k: int, seed: int = 1007, n_pad: int = 0, n_dup: int = 0,
              n_out: int = 0) -> np.ndarray:
    """An int32 row list like a top-k selection over T cached rows: k distinct
    rows in random (not sorted) order, then n_dup repeats of listed rows at
    random places, n_out entries naming rows past the cache, and n_pad
    entries of -1 at the end (a fixed-size selection buffer that is not
    full).  Rows are drawn uniformly: which rows win does not change the work."""
    g = rng(seed)
    sel = g.permutation(T)[:k].astype(np.int64)
    if n_dup:
        at = g.integers(0, sel.size + 1, n_dup)
        sel = np.insert(sel, np.sort(at), g.choice(sel[:k], n_dup))
    if n_out:
        at = g.integers(0, sel.size + 1, n_out)
        sel = np.insert(sel, np.sort(at), T + g.integers(0, 1 << 20, n_out))
    sel = np.concatenate([sel, np.full(n_pad, -1, np.int64)])
    return sel.astype(np.int32)
