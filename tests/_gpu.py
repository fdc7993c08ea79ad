"""Helpers for the GPU parity tests: device transfer and case announcements."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a failing run names it."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return host(t).view(np.uint16)


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got.view(np.uint8), want.view(np.uint8)):
        bad = np.nonzero(got.reshape(-1).view(np.uint8) != want.reshape(-1).view(np.uint8))[0]
        raise AssertionError(f"{what}: {bad.size} differing bytes, first at {bad[:8].tolist()}")


ATTN_TOL = 1e-5
# Per query row the bar is ATTN_TOL, or F32_ROW_FACTOR times the error that a
# plain float32 evaluation of the same formulas makes on that row, whichever
# is larger.  A row whose output is small next to the values it averages
# (heavy cancellation), or whose softmax weights hinge on scores of large
# magnitude, cannot be computed to 1e-5 of itself with float32 scores and
# sums: the float32 twin of the oracle shows how far such a row moves from
# rounding alone.
F32_ROW_FACTOR = 4.0


def reference(fn, *args, **kw):
    """The oracle's float64 result (out, lse) of attention function fn, and
    the same formulas evaluated in float32 (out only) for the per-row bar."""
    import numpy as np
    ro, rl = fn(*args, **kw)
    tw, _ = fn(*args, dtype=np.float32, **kw)
    return ro, rl, tw


def row_rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Relative L2 error of each query row (rows along the first axis); a row
    whose reference is exactly zero scores its own norm (0 when it is 0)."""
    g = np.asarray(got, np.float64).reshape(len(ref), -1)
    r = np.asarray(ref, np.float64).reshape(len(ref), -1)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def check_attention(out, lse, ref_out, ref_lse, what: str, tol: float = ATTN_TOL, twin=None) -> None:
    """The attention bar: relative L2 over the whole output within tol; every
    query row on its own within max(tol, F32_ROW_FACTOR x the float32 twin's
    error on that row) (so one head cannot hide behind the others); lse
    within tol * max(1, |lse|) per element."""
    from oracle import kvq_oracle as o
    out = np.asarray(out)
    ref_out = np.asarray(ref_out)
    r = o.rel_l2(out, ref_out)
    rows = row_rel_l2(out, ref_out)
    bar = np.full(rows.shape, tol)
    if twin is not None:
        e32 = row_rel_l2(np.asarray(twin, np.float64).reshape(ref_out.shape), ref_out)
        bar = np.maximum(bar, F32_ROW_FACTOR * e32)
    ratio = rows / bar
    worst = int(np.argmax(ratio))
    msg = (f"  {what}: rel_l2={r:.3e} worst_row={rows.max():.3e} (row {int(np.argmax(rows))}); "
           f"tightest row {worst}: {rows[worst]:.3e} vs bar {bar[worst]:.3e}")
    if lse is not None:
        lse = np.asarray(lse, np.float64).reshape(-1)
        ref_lse = np.asarray(ref_lse, np.float64).reshape(-1)
        with np.errstate(invalid="ignore"):
            same_inf = np.isinf(ref_lse) & (lse == ref_lse)
            rel = np.abs(lse - ref_lse) / np.maximum(1.0, np.abs(ref_lse))
        rl = float(np.max(np.where(same_inf, 0.0, rel)))
        msg += f" lse_err={rl:.3e}"
    print(msg, flush=True)
    assert r <= tol, (what, "whole tensor", r)
    assert ratio[worst] <= 1.0, (what, "query row", worst, rows[worst], bar[worst])
    if lse is not None:
        assert rl <= tol, (what, "lse", rl)
