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
