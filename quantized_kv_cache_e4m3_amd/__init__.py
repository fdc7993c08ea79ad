"""Python binding of libkvq.so (quantized KV-cache encoders and attention for
gfx950).  Argument marshalling only: every step runs in the library's HIP
kernels, on the caller's current torch stream.  There is no fallback: if the
library is missing the import fails.

The functions keep the C names (see include/kvq.h):
    kv_encode_fp8, kv_encode_tq4, kv_encode_q2k, kv_append_q2k, q2k_alloc,
    attn_decode_quant, attn_decode_quant_noalloc, attn_prefill_quant,
    attn_workspace_bytes, attn_decode_gather, attn_gather_workspace_bytes,
    kvq_row_bytes, kvq_codebook, kvq_status_str
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

KVQ_FP8, KVQ_TQ4, KVQ_Q2K = 1, 2, 3
KVQ_ERR_SCRATCH = 7
NOALLOC_SCRATCH_BYTES = 16 << 20      # KVQ_NOALLOC_SCRATCH_BYTES
FORMATS = {"fp8": KVQ_FP8, "tq4": KVQ_TQ4, "q2k": KVQ_Q2K}


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {kvq_status_str(status)} (status {status})")
        self.status = status


class KvqCacheStruct(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("n_kv", ctypes.c_int32),
        ("n_sink", ctypes.c_int32),
        ("n_window", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("n_rows", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("v_blocks", ctypes.c_void_p),
        ("k_ovl", ctypes.c_void_p),
        ("v_ovl", ctypes.c_void_p),
        ("rot_seed", ctypes.c_uint64),
        ("rope_codes", ctypes.c_void_p),
        ("rope_scales", ctypes.c_void_p),
        ("rope_seed", ctypes.c_uint64),
        ("n_slack", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python quantized_kv_cache_e4m3_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_float, ctypes.c_size_t)
    cp = ctypes.POINTER(KvqCacheStruct)
    sig = {
        "kv_encode_fp8": (i32, [vp, i64, i32, vp, vp, vp]),
        "kv_encode_tq4": (i32, [vp, i64, i32, u64, vp, vp, vp]),
        "kv_encode_q2k": (i32, [vp, vp, i64, i32, i32, f32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "kv_append_q2k": (i32, [vp, vp, i64, i64, i32, i32, f32, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "attn_workspace_bytes": (sz, [cp, i32, i32]),
        "attn_decode_quant": (i32, [cp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "attn_decode_quant_noalloc": (i32, [cp, vp, i32, f32, vp, vp, vp]),
        "attn_decode_append_fp8": (i32, [cp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "attn_prefill_quant": (i32, [cp, vp, i32, i32, i64, f32, vp, vp, vp, sz, vp]),
        "attn_gather_workspace_bytes": (sz, [cp, i32, i64]),
        "attn_decode_gather": (i32, [cp, vp, i64, vp, i32, f32, vp, vp, vp, sz, vp]),
        "kvq_row_bytes": (sz, [i32, i32, i32]),
        "kvq_codebook": (i32, [i32, vp]),
        "kvq_status_str": (ctypes.c_char_p, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()
EXPORTED = ("kv_encode_fp8", "kv_encode_tq4", "kv_encode_q2k", "kv_append_q2k", "attn_workspace_bytes",
            "attn_decode_quant", "attn_decode_quant_noalloc", "attn_decode_append_fp8", "attn_prefill_quant",
            "attn_gather_workspace_bytes", "attn_decode_gather", "kvq_row_bytes", "kvq_codebook", "kvq_status_str")


def kvq_status_str(status: int) -> str:
    return lib.kvq_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KvqError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensors only")
    if not t.is_contiguous():
        raise ValueError("contiguous tensors only")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, dtype, shape, name):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def kvq_row_bytes(fmt, d: int, n_kv: int = 1) -> int:
    return int(lib.kvq_row_bytes(FORMATS.get(fmt, fmt), d, n_kv))


def kvq_codebook(levels: int):
    buf = (ctypes.c_float * levels)()
    _check(lib.kvq_codebook(levels, ctypes.cast(buf, ctypes.c_void_p)), "kvq_codebook")
    return list(buf)


# ---------------------------------------------------------------------------
# encoders
# ---------------------------------------------------------------------------

def kv_encode_fp8(x, codes=None, scales=None, stream=None):
    """x f32 [n, d] -> (codes u8 [n, d], scales f32 [n])."""
    n, d = x.shape
    if codes is None:
        codes = torch.empty((n, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((n,), dtype=torch.float32, device=x.device)
    _need(x, torch.float32, (n, d), "x")
    _need(codes, torch.uint8, (n, d), "codes")
    _need(scales, torch.float32, (n,), "scales")
    _check(lib.kv_encode_fp8(_ptr(x), n, d, _ptr(codes), _ptr(scales), _stream(stream)),
           "kv_encode_fp8")
    return codes, scales


def kv_encode_tq4(x, rot_seed: int, packed=None, radius=None, stream=None):
    """x f32 [n, d] -> (packed u8 [n, d/2], radius f32 [n])."""
    n, d = x.shape
    if packed is None:
        packed = torch.empty((n, d // 2), dtype=torch.uint8, device=x.device)
    if radius is None:
        radius = torch.empty((n,), dtype=torch.float32, device=x.device)
    _need(x, torch.float32, (n, d), "x")
    _need(packed, torch.uint8, (n, d // 2), "packed")
    _need(radius, torch.float32, (n,), "radius")
    _check(lib.kv_encode_tq4(_ptr(x), n, d, int(rot_seed) & (2 ** 64 - 1), _ptr(packed), _ptr(radius),
                             _stream(stream)), "kv_encode_tq4")
    return packed, radius


def kv_encode_q2k(k, v, k_gain: float, n_sink: int, n_window: int, out=None, stream=None):
    """k, v f32 [T, n_kv, d] -> dict(k_codes, k_scale, v_blocks, k_ovl, v_ovl)."""
    T, n_kv, d = k.shape
    dev = k.device
    if out is None:
        out = {
            "k_codes": torch.empty((T // 32, n_kv, d, 8), dtype=torch.uint8, device=dev),
            "k_scale": torch.empty((T // 32, n_kv, d), dtype=torch.int16, device=dev),
            "v_blocks": torch.empty((T, n_kv, d // 32, 18), dtype=torch.uint8, device=dev),
            "k_ovl": torch.empty((n_sink + n_window, n_kv, d), dtype=torch.int16, device=dev)
            if n_sink + n_window > 0 else None,
            "v_ovl": torch.empty((n_sink + n_window, n_kv, d), dtype=torch.int16, device=dev)
            if n_sink + n_window > 0 else None,
        }
    _need(k, torch.float32, (T, n_kv, d), "k")
    _need(v, torch.float32, (T, n_kv, d), "v")
    _check(lib.kv_encode_q2k(_ptr(k), _ptr(v), T, n_kv, d, float(k_gain), n_sink, n_window,
                             _ptr(out["k_codes"]), _ptr(out["k_scale"]), _ptr(out["v_blocks"]),
                             _ptr(out["k_ovl"]), _ptr(out["v_ovl"]), _stream(stream)),
           "kv_encode_q2k")
    return out


def q2k_alloc(cap_cells: int, n_kv: int, d: int, n_sink: int, n_window: int, n_slack: int = 16,
              device="cuda:0"):
    """Zeroed q2k buffers for up to cap_cells cells, filled by kv_append_q2k."""
    G = (cap_cells + 31) // 32
    n_ovl = n_sink + n_window + n_slack
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
    return {
        "k_codes": z((G, n_kv, d, 8), torch.uint8),
        "k_scale": z((G, n_kv, d), torch.int16),
        "v_blocks": z((G * 32, n_kv, d // 32, 18), torch.uint8),
        "k_ovl": z((n_ovl, n_kv, d), torch.int16) if n_sink + n_window > 0 else None,
        "v_ovl": z((n_ovl, n_kv, d), torch.int16) if n_sink + n_window > 0 else None,
    }


def kv_append_q2k(k, v, n_prev: int, k_gain: float, n_sink: int, n_window: int, n_slack: int,
                  out, stream=None):
    """Append cells [n_prev, len(k)) of k, v (f32 [n, n_kv, d], every cell so
    far) to the q2k buffers `out` (from q2k_alloc); returns out."""
    T, n_kv, d = k.shape
    _need(k, torch.float32, (T, n_kv, d), "k")
    _need(v, torch.float32, (T, n_kv, d), "v")
    if not 0 <= n_prev <= T:
        raise ValueError("n_prev must lie in [0, len(k)]")
    if out["k_codes"].shape[0] * 32 < T or out["v_blocks"].shape[0] < 32 * ((T + 31) // 32):
        raise ValueError("q2k buffers too small for the appended cells")
    if n_sink + n_window > 0 and (out["k_ovl"] is None or out["v_ovl"] is None or
                                  out["k_ovl"].shape[0] < n_sink + n_window + n_slack or
                                  out["v_ovl"].shape[0] < n_sink + n_window + n_slack):
        raise ValueError("overlay buffers need n_sink + n_window + n_slack slots")
    _check(lib.kv_append_q2k(_ptr(k), _ptr(v), int(n_prev), int(T - n_prev), n_kv, d, float(k_gain),
                             n_sink, n_window, n_slack, _ptr(out["k_codes"]), _ptr(out["k_scale"]),
                             _ptr(out["v_blocks"]), _ptr(out["k_ovl"]), _ptr(out["v_ovl"]),
                             _stream(stream)), "kv_append_q2k")
    return out


# ---------------------------------------------------------------------------
# caches and attention
# ---------------------------------------------------------------------------

class Cache:
    """Holds the device tensors of one encoded cache and its kvq_cache view."""

    def __init__(self, fmt, d, n_rows, codes, scales, n_kv=1, v_blocks=None, k_ovl=None,
                 v_ovl=None, n_sink=0, n_window=0, rot_seed=0, d_rope=0, rope_codes=None,
                 rope_scales=None, rope_seed=0, n_slack=0):
        self.tensors = (codes, scales, v_blocks, k_ovl, v_ovl, rope_codes, rope_scales)  # keep alive
        self.fmt = FORMATS.get(fmt, fmt)
        self.d, self.d_rope = d, d_rope
        self.struct = KvqCacheStruct(
            fmt=self.fmt, d=d, n_kv=n_kv, n_sink=n_sink, n_window=n_window, d_rope=d_rope,
            n_rows=n_rows, codes=_ptr(codes), scales=_ptr(scales), v_blocks=_ptr(v_blocks),
            k_ovl=_ptr(k_ovl), v_ovl=_ptr(v_ovl), rot_seed=int(rot_seed) & (2 ** 64 - 1),
            rope_codes=_ptr(rope_codes), rope_scales=_ptr(rope_scales),
            rope_seed=int(rope_seed) & (2 ** 64 - 1), n_slack=n_slack, reserved=0)

    @property
    def ref(self):
        return ctypes.byref(self.struct)

    @classmethod
    def fp8(cls, codes, scales, rope=None):
        """rope: optional (rope_codes, rope_scales) from kv_encode_fp8 of the rope rows."""
        if rope is None:
            return cls("fp8", codes.shape[1], codes.shape[0], codes, scales)
        rc, rs = rope
        return cls("fp8", codes.shape[1], codes.shape[0], codes, scales, d_rope=rc.shape[1],
                   rope_codes=rc, rope_scales=rs)

    @classmethod
    def tq4(cls, packed, radius, rot_seed, rope=None):
        """rope: optional (rope_packed, rope_radius, rope_seed) from kv_encode_tq4 of the rope rows."""
        if rope is None:
            return cls("tq4", packed.shape[1] * 2, packed.shape[0], packed, radius, rot_seed=rot_seed)
        rp, rr, rseed = rope
        return cls("tq4", packed.shape[1] * 2, packed.shape[0], packed, radius, rot_seed=rot_seed,
                   d_rope=rp.shape[1] * 2, rope_codes=rp, rope_scales=rr, rope_seed=rseed)

    @classmethod
    def q2k(cls, enc, n_sink, n_window, n_slack=0, n_cells=None):
        """enc: buffers from kv_encode_q2k or q2k_alloc + kv_append_q2k;
        n_cells: cells present (default: every cell of the groups)."""
        kc = enc["k_codes"]
        G, n_kv, d, _ = kc.shape
        return cls("q2k", d, G * 32 if n_cells is None else n_cells, kc, enc["k_scale"], n_kv=n_kv,
                   v_blocks=enc["v_blocks"], k_ovl=enc["k_ovl"], v_ovl=enc["v_ovl"],
                   n_sink=n_sink, n_window=n_window, n_slack=n_slack)


def attn_workspace_bytes(cache: Cache, n_q_heads: int, n_query_tokens: int = 1) -> int:
    return int(lib.attn_workspace_bytes(cache.ref, n_q_heads, n_query_tokens))


def _workspace(cache, n_q_heads, S, ws, device):
    need = attn_workspace_bytes(cache, n_q_heads, S)
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=device)
    return ws


def attn_decode_quant(cache: Cache, q, sm_scale: float, out=None, lse=None, ws=None, stream=None,
                      want_lse: bool = True):
    """q f32 [Hq, d + d_rope] -> (out f32 [Hq, d], lse f32 [Hq] or None)."""
    Hq = q.shape[0]
    d = cache.d
    _need(q, torch.float32, (Hq, d + cache.d_rope), "q")
    if out is None:
        out = torch.empty((Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
    ws = _workspace(cache, Hq, 1, ws, q.device)
    _check(lib.attn_decode_quant(cache.ref, _ptr(q), Hq, float(sm_scale), _ptr(out), _ptr(lse),
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "attn_decode_quant")
    return out, lse


def attn_decode_quant_noalloc(cache: Cache, q, sm_scale: float, out=None, lse=None, stream=None,
                              want_lse: bool = True):
    """attn_decode_quant with the library's per-GPU scratch in place of a
    workspace (out / lse are allocated here only when not given)."""
    Hq = q.shape[0]
    d = cache.d
    _need(q, torch.float32, (Hq, d + cache.d_rope), "q")
    if out is None:
        out = torch.empty((Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
    _check(lib.attn_decode_quant_noalloc(cache.ref, _ptr(q), Hq, float(sm_scale), _ptr(out), _ptr(lse),
                                         _stream(stream)), "attn_decode_quant_noalloc")
    return out, lse


def attn_decode_append_fp8(cache: Cache, x_new, q, sm_scale: float, out=None, lse=None, ws=None,
                           stream=None, want_lse: bool = True):
    """One decode step of an FP8 cache whose last row is new: x_new f32 [d] is
    encoded into that row (cache.tensors' codes / scales), then
    q f32 [Hq, d + d_rope] attends every row -> (out f32 [Hq, d], lse or None)."""
    Hq = q.shape[0]
    d = cache.d
    if cache.fmt != KVQ_FP8:
        raise ValueError("attn_decode_append_fp8: FP8 caches only")
    _need(x_new, torch.float32, (d,), "x_new")
    _need(q, torch.float32, (Hq, d + cache.d_rope), "q")
    codes, scales = cache.tensors[0], cache.tensors[1]
    if out is None:
        out = torch.empty((Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
    ws = _workspace(cache, Hq, 1, ws, q.device)
    _check(lib.attn_decode_append_fp8(cache.ref, _ptr(x_new), _ptr(codes), _ptr(scales), _ptr(q), Hq,
                                      float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "attn_decode_append_fp8")
    return out, lse


def attn_prefill_quant(cache: Cache, q, pos0: int, sm_scale: float, out=None, lse=None, ws=None,
                       stream=None, want_lse: bool = True):
    """q f32 [S, Hq, d + d_rope] -> (out f32 [S, Hq, d], lse f32 [S, Hq] or None)."""
    S, Hq = q.shape[0], q.shape[1]
    d = cache.d
    _need(q, torch.float32, (S, Hq, d + cache.d_rope), "q")
    if out is None:
        out = torch.empty((S, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    ws = _workspace(cache, Hq, S, ws, q.device)
    _check(lib.attn_prefill_quant(cache.ref, _ptr(q), S, Hq, int(pos0), float(sm_scale), _ptr(out),
                                  _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "attn_prefill_quant")
    return out, lse


def attn_gather_workspace_bytes(cache: Cache, n_q_heads: int, n_idx: int) -> int:
    return int(lib.attn_gather_workspace_bytes(cache.ref, n_q_heads, int(n_idx)))


def attn_decode_gather(cache: Cache, idx, q, sm_scale: float, out=None, lse=None, ws=None,
                       stream=None, want_lse: bool = True):
    """idx i32 [n] (absolute cache rows; outside [0, n_rows) = padding),
    q f32 [Hq, d + d_rope] -> (out f32 [Hq, d], lse f32 [Hq] or None)."""
    Hq = q.shape[0]
    d = cache.d
    n = idx.numel()
    _need(idx, torch.int32, (n,), "idx")
    _need(q, torch.float32, (Hq, d + cache.d_rope), "q")
    if out is None:
        out = torch.empty((Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((Hq,), dtype=torch.float32, device=q.device)
    if ws is None:
        need = attn_gather_workspace_bytes(cache, Hq, n)
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=q.device)
    _check(lib.attn_decode_gather(cache.ref, _ptr(idx), n, _ptr(q), Hq, float(sm_scale), _ptr(out),
                                  _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)), "attn_decode_gather")
    return out, lse
