"""Range-masked ("flex") flash attention on MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/ffa.h``.  Every step of the
computation (planning, kernels) runs in the native library; this module only
marshals arguments: torch tensors supply device memory and the current HIP
stream.  If the library is not built the functions raise; there is no
fallback implementation.

``flex_flash_attn_func`` mirrors the call in the MagiAttention issue "Using
dummy/padded attention slices with flex_flash_attn_func for torch.compile
static shapes" (q, k, v packed as [tokens, heads, head_dim]; int32 q_ranges,
k_ranges [R, 2] and attn_type_map [R] with 0 = FULL, 1 = CAUSAL;
softmax_scale None = 1/sqrt(head_dim); softcap 0 = off) and returns
``(out, lse)``; it supports autograd.
"""
from __future__ import annotations

import collections
import ctypes
import math
import os
import threading
from typing import Optional, Tuple

import numpy as np

__all__ = [
    "FULL", "CAUSAL", "FfaError", "lib_path", "load_library", "ffa_fwd", "ffa_bwd",
    "ffa_bwd_workspace_size", "ffa_plan_host", "ffa_last_error", "ffa_build_info",
    "ffa_plan_create", "ffa_fwd_planned", "ffa_bwd_planned", "ffa_plan_destroy",
    "ffa_plan_device_workspace_size", "ffa_plan_create_device", "ffa_plan_refresh", "ffa_plan_status",
    "ffa_plan_export", "FFA_PLAN_BAD_SLICE", "FFA_PLAN_CAPACITY", "flex_flash_attn_func",
    "alibi_geometric_slopes", "ffa_block_slices", "cached_plan", "clear_plan_cache", "ffa_fwd_ex", "ffa_bwd_ex", "ffa_saved_size", "ffa_fwd_noalloc", "ffa_fwd_planned_ex", "ffa_bwd_planned_ex",
]

FULL = 0
CAUSAL = 1

_STATUS = {0: "FFA_OK", -1: "FFA_ERR_INVALID_ARG", -2: "FFA_ERR_UNSUPPORTED",
           -3: "FFA_ERR_HIP", -4: "FFA_ERR_NOMEM"}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FfaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_STATUS.get(code, code)}: {msg}")
        self.code = code


def lib_path() -> str:
    return os.path.join(_PKG, "_lib", "libffa.so")


def load_library():
    """Load the native library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = lib_path()
    if not os.path.exists(p):
        raise RuntimeError(f"native library missing: {p} (build it with "
                           "`python -m range_masked_attention_amd._build`)")
    lib = ctypes.CDLL(p)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    ip32 = ctypes.POINTER(ctypes.c_int32)
    lib.ffa_fwd.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, ip32, ip32, ip32, i32,
                            f32, f32, vp, vp, vp]
    lib.ffa_fwd.restype = ctypes.c_int
    lib.ffa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ip32, ip32, ip32,
                            i32, f32, f32, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ffa_bwd.restype = ctypes.c_int
    lib.ffa_fwd_noalloc.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, ip32, ip32, ip32, i32,
                                    f32, f32, vp, vp, vp]
    lib.ffa_fwd_noalloc.restype = ctypes.c_int
    lib.ffa_fwd_ex.argtypes = [vp, vp, vp, i64, i64, i32, i32, i32, ip32, ip32, ip32, i32,
                               f32, f32, vp, vp, vp, vp, vp]
    lib.ffa_fwd_ex.restype = ctypes.c_int
    lib.ffa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, ip32, ip32, ip32,
                               i32, f32, f32, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ffa_bwd_ex.restype = ctypes.c_int
    lib.ffa_saved_size.argtypes = [i64, i64, i32, i32, i32]
    lib.ffa_saved_size.restype = ctypes.c_size_t
    lib.ffa_bwd_workspace_size.argtypes = [i64, i64, i32, i32, i32]
    lib.ffa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.ffa_plan_host.argtypes = [i64, i64, ip32, ip32, ip32, i32, i32, i32, i32,
                                  ctypes.POINTER(ctypes.c_int64), ip32, i64, ip32]
    lib.ffa_plan_host.restype = ctypes.c_int64
    lib.ffa_block_slices.argtypes = [i64, i64, i32, i32, ip32, ip32, i32, ip32, ip32, ip32, i64]
    lib.ffa_block_slices.restype = ctypes.c_int64
    lib.ffa_plan_create.argtypes = [i64, i64, ip32, ip32, ip32, i32, vp, ctypes.POINTER(vp)]
    lib.ffa_plan_create.restype = ctypes.c_int
    lib.ffa_fwd_planned.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp]
    lib.ffa_fwd_planned.restype = ctypes.c_int
    lib.ffa_bwd_planned.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, f32,
                                    vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ffa_bwd_planned.restype = ctypes.c_int
    lib.ffa_fwd_planned_ex.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, f32, vp, vp, vp, vp, vp]
    lib.ffa_fwd_planned_ex.restype = ctypes.c_int
    lib.ffa_bwd_planned_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, f32, vp,
                                       vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.ffa_bwd_planned_ex.restype = ctypes.c_int
    lib.ffa_plan_destroy.argtypes = [vp, vp]
    lib.ffa_plan_destroy.restype = ctypes.c_int
    lib.ffa_plan_device_workspace_size.argtypes = [i64, i64, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.ffa_plan_device_workspace_size.restype = ctypes.c_int
    lib.ffa_plan_create_device.argtypes = [i64, i64, vp, vp, vp, i32, i64, vp, ctypes.c_size_t, vp,
                                           ctypes.POINTER(vp)]
    lib.ffa_plan_create_device.restype = ctypes.c_int
    lib.ffa_plan_refresh.argtypes = [vp, vp]
    lib.ffa_plan_refresh.restype = ctypes.c_int
    lib.ffa_plan_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int)]
    lib.ffa_plan_status.restype = ctypes.c_int
    lib.ffa_plan_export.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                    ip32, i64, ip32, vp]
    lib.ffa_plan_export.restype = ctypes.c_int64
    lib.ffa_last_error.restype = ctypes.c_char_p
    lib.ffa_build_info.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def ffa_last_error() -> str:
    return load_library().ffa_last_error().decode()


def ffa_build_info() -> str:
    return load_library().ffa_build_info().decode()


def _check(rc: int):
    if rc != 0:
        raise FfaError(rc, ffa_last_error())


def _host_slices(q_ranges, k_ranges, attn_type_map):
    """Slice arrays as contiguous host int32 (device tensors are copied: one sync)."""
    def to_np(x, shape_tail):
        if hasattr(x, "detach"):
            x = x.detach().cpu().numpy()
        a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
        return a.reshape((-1,) + shape_tail)
    qr = to_np(q_ranges, (2,))
    kr = to_np(k_ranges, (2,))
    ty = to_np(attn_type_map, ())
    if not (qr.shape[0] == kr.shape[0] == ty.shape[0]):
        raise ValueError("q_ranges, k_ranges and attn_type_map must have the same number of rows")
    return qr, kr, ty


def _iptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _stream_handle(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_tensor(name, t, dtype, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def alibi_geometric_slopes(hq: int):
    """ALiBi's geometric head slopes 2^(-8 h / hq), h = 1 .. hq, as a list.

    Pass them (as an fp32 tensor on the GPU) to the ``alibi_slopes`` argument,
    which adds ``slope[h] * (j - i)`` to the scores: with positive slopes on a
    causal mask, a penalty growing linearly with the distance i - j.
    """
    return [2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)]


def _slopes_ptr(slopes, hq: int, device):
    """Device pointer of an fp32 [hq] slope tensor, or None."""
    import torch
    if slopes is None:
        return None
    if not isinstance(slopes, torch.Tensor):
        raise TypeError("alibi_slopes must be a torch.Tensor (fp32 [hq] on the GPU)")
    if slopes.dtype != torch.float32 or tuple(slopes.shape) != (hq,):
        raise ValueError(f"alibi_slopes must be fp32 of shape ({hq},), got {slopes.dtype} {tuple(slopes.shape)}")
    if not slopes.is_cuda or slopes.device != device or not slopes.is_contiguous():
        raise ValueError("alibi_slopes must be a contiguous tensor on the inputs' GPU")
    return slopes.data_ptr()


def ffa_saved_size(Tq: int, Tk: int, hq: int, hkv: int, d: int) -> int:
    """C ABI ``ffa_saved_size``: bytes of the training forward's saved record."""
    return int(load_library().ffa_saved_size(Tq, Tk, hq, hkv, d))


def _saved_tensor(saved, train, q, k):
    """The saved record to use: the caller's uint8 tensor, a new one (train=True), or None."""
    import torch
    need = ffa_saved_size(q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2])
    if saved is None and train:
        saved = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if saved is not None:
        if not isinstance(saved, torch.Tensor) or saved.dtype != torch.uint8 or not saved.is_cuda \
                or not saved.is_contiguous():
            raise TypeError("saved must be a contiguous uint8 tensor on the GPU")
        if saved.numel() < need:
            raise ValueError(f"saved needs {need} bytes (ffa_saved_size), got {saved.numel()}")
    return saved


def ffa_fwd(q, k, v, q_ranges, k_ranges, attn_type_map, scale: float, softcap: float = 0.0,
            out=None, lse=None, alibi_slopes=None, saved=None, train: bool = False):
    """C ABI ``ffa_fwd`` (``ffa_fwd_ex`` with ``alibi_slopes`` or a saved record) on torch tensors.

    Returns (out [Tq,hq,d] bf16, lse [Tq,hq] fp32); with ``train=True`` or a
    ``saved`` tensor (uint8, ``ffa_saved_size`` bytes) it runs the training
    forward, which fills the record for ``ffa_bwd``, and returns it third.
    """
    import torch
    lib = load_library()
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(nm, t, torch.bfloat16, 3)
    Tq, hq, d = q.shape
    Tk, hkv, _ = k.shape
    if tuple(v.shape) != tuple(k.shape) or k.shape[2] != d:
        raise ValueError("k and v must both be [Tk, hkv, d] with q's head_dim")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Tq, hq), dtype=torch.float32, device=q.device)
    _check_tensor("out", out, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (Tq, hq):
        raise ValueError("out must be shaped like q and lse [Tq, hq]")
    saved = _saved_tensor(saved, train, q, k)
    qr, kr, ty = _host_slices(q_ranges, k_ranges, attn_type_map)
    sp = _slopes_ptr(alibi_slopes, hq, q.device)
    head = (q.data_ptr(), k.data_ptr(), v.data_ptr(), Tq, Tk, hq, hkv, d,
            _iptr(qr), _iptr(kr), _iptr(ty), qr.shape[0], float(scale), float(softcap))
    st = _stream_handle(q)
    if sp is None and saved is None:
        rc = lib.ffa_fwd(*head, out.data_ptr(), lse.data_ptr(), st)
    else:
        rc = lib.ffa_fwd_ex(*head, sp, out.data_ptr(), lse.data_ptr(),
                            saved.data_ptr() if saved is not None else None, st)
    _check(rc)
    return (out, lse) if saved is None else (out, lse, saved)


def ffa_fwd_noalloc(q, k, v, q_ranges, k_ranges, attn_type_map, scale: float, softcap: float, out, lse):
    """C ABI ``ffa_fwd_noalloc``: ``ffa_fwd`` into the caller's ``out`` and ``lse``
    with no device allocation (the library's own device array holds the plan)."""
    import torch
    lib = load_library()
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(nm, t, torch.bfloat16, 3)
    _check_tensor("out", out, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    Tq, hq, d = q.shape
    Tk, hkv, _ = k.shape
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (Tq, hq):
        raise ValueError("out must be shaped like q and lse [Tq, hq]")
    qr, kr, ty = _host_slices(q_ranges, k_ranges, attn_type_map)
    _check(lib.ffa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), Tq, Tk, hq, hkv, d,
                               _iptr(qr), _iptr(kr), _iptr(ty), qr.shape[0], float(scale), float(softcap),
                               out.data_ptr(), lse.data_ptr(), _stream_handle(q)))
    return out, lse


def ffa_bwd_workspace_size(Tq: int, Tk: int, hq: int, hkv: int, d: int) -> int:
    """C ABI ``ffa_bwd_workspace_size``: bytes of device workspace the backward needs."""
    return int(load_library().ffa_bwd_workspace_size(Tq, Tk, hq, hkv, d))


def ffa_bwd(q, k, v, out, lse, dout, q_ranges, k_ranges, attn_type_map, scale: float,
            softcap: float = 0.0, dq=None, dk=None, dv=None, workspace=None, alibi_slopes=None,
            saved=None):
    """C ABI ``ffa_bwd`` (``ffa_bwd_ex`` with ``alibi_slopes`` or ``saved``) on torch tensors.

    ``saved``: the record a training forward (``train=True``) filled; without
    it the library re-runs the training forward to get one.  Returns (dq, dk,
    dv) in bf16.
    """
    import torch
    lib = load_library()
    for nm, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(nm, t, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    Tq, hq, d = q.shape
    Tk, hkv, _ = k.shape
    if tuple(out.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("out and dout must be shaped like q")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for nm, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(nm, t, torch.bfloat16, 3)
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{nm} must be shaped like its input")
    ws_bytes = ffa_bwd_workspace_size(Tq, Tk, hq, hkv, d)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    saved = _saved_tensor(saved, False, q, k)
    qr, kr, ty = _host_slices(q_ranges, k_ranges, attn_type_map)
    sp = _slopes_ptr(alibi_slopes, hq, q.device)
    sizes = (Tq, Tk, hq, hkv, d, _iptr(qr), _iptr(kr), _iptr(ty), qr.shape[0], float(scale), float(softcap))
    tail = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_len, _stream_handle(q))
    qkv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    if sp is None and saved is None:
        rc = lib.ffa_bwd(*qkv, dout.data_ptr(), *sizes, *tail)
    else:
        rc = lib.ffa_bwd_ex(*qkv, saved.data_ptr() if saved is not None else None, dout.data_ptr(),
                            *sizes, sp, *tail)
    _check(rc)
    return dq, dk, dv


def ffa_plan_host(Tq: int, Tk: int, q_ranges, k_ranges, attn_type_map, bm: int, bn: int,
                  transpose: bool = False):
    """C ABI ``ffa_plan_host``: (row_ptr [n+1] int64, entries [E,3] int32, order [n] int32)."""
    lib = load_library()
    qr, kr, ty = _host_slices(q_ranges, k_ranges, attn_type_map)
    args = (Tq, Tk, _iptr(qr), _iptr(kr), _iptr(ty), qr.shape[0], bm, bn, int(bool(transpose)))
    n = lib.ffa_plan_host(*args, None, None, 0, None)
    if n < 0:
        raise FfaError(int(n), ffa_last_error())
    n_tiles = -(-(Tk if transpose else Tq) // (bn if transpose else bm))
    row_ptr = np.zeros(n_tiles + 1, dtype=np.int64)
    entries = np.zeros((max(n, 1), 3), dtype=np.int32)
    order = np.zeros(max(n_tiles, 1), dtype=np.int32)
    n2 = lib.ffa_plan_host(*args, row_ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                           _iptr(entries), n, _iptr(order))
    if n2 != n:
        raise FfaError(int(n2), ffa_last_error())
    return row_ptr, entries[:n], order[:n_tiles]


def ffa_block_slices(kv_num_blocks, kv_indices, Tq: int, Tk: int, block_q: int = 128,
                     block_k: int = 128):
    """C ABI ``ffa_block_slices``: FULL slices covering a BlockMask-style block list.

    ``kv_num_blocks`` [n_qblocks] and ``kv_indices`` [n_qblocks, max_blocks]
    (host arrays or tensors, int32-convertible): query block b sees the key
    blocks ``kv_indices[b, :kv_num_blocks[b]]``.  Returns (q_ranges [R, 2],
    k_ranges [R, 2], attn_type_map [R]) as int32 NumPy arrays.
    """
    lib = load_library()

    def host(x):
        if hasattr(x, "detach"):
            x = x.detach().cpu().numpy()
        return np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    num = host(kv_num_blocks).reshape(-1)
    idx = host(kv_indices)
    idx = idx.reshape(num.shape[0], -1) if idx.size else np.zeros((num.shape[0], 0), np.int32)
    width = idx.shape[1]
    args = (Tq, Tk, block_q, block_k, _iptr(num), _iptr(idx), width)
    n = lib.ffa_block_slices(*args, None, None, None, 0)
    if n < 0:
        raise FfaError(int(n), ffa_last_error())
    qr = np.zeros((n, 2), np.int32)
    kr = np.zeros((n, 2), np.int32)
    ty = np.zeros(n, np.int32)
    n2 = lib.ffa_block_slices(*args, _iptr(qr), _iptr(kr), _iptr(ty), n)
    if n2 != n:
        raise FfaError(int(n2), ffa_last_error())
    return qr, kr, ty


def ffa_plan_create(Tq: int, Tk: int, q_ranges, k_ranges, attn_type_map, device=None) -> int:
    """C ABI ``ffa_plan_create`` on the current stream of ``device``; returns the handle."""
    import torch
    lib = load_library()
    qr, kr, ty = _host_slices(q_ranges, k_ranges, attn_type_map)
    dev_ = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    h = ctypes.c_void_p()
    rc = lib.ffa_plan_create(Tq, Tk, _iptr(qr), _iptr(kr), _iptr(ty), qr.shape[0],
                             torch.cuda.current_stream(dev_).cuda_stream, ctypes.byref(h))
    _check(rc)
    return h.value


def ffa_plan_destroy(plan, device=None) -> None:
    """C ABI ``ffa_plan_destroy`` (stream-ordered on the current stream)."""
    import torch
    if plan is None:
        return
    dev_ = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    _check(load_library().ffa_plan_destroy(plan, torch.cuda.current_stream(dev_).cuda_stream))


class _PlanCache:
    """Plans of recently seen slice lists, per (device, stream, Tq, Tk, slices).

    A plan depends only on the sizes and the slice list, so layers and steps
    that share a mask can share it: the host planning and upload then happen
    once instead of on every call.  Keyed by stream as well, because a plan is
    uploaded on its stream and its forward scratch must not be used by two
    streams at once.  Least recently used plans are destroyed, in order, on
    the stream they were made for.
    """

    def __init__(self, capacity: int):
        self.capacity = capacity
        self._plans = collections.OrderedDict()
        self._lock = threading.Lock()
        self.hits = 0
        self.misses = 0

    def get(self, Tq: int, Tk: int, q_ranges, k_ranges, attn_type_map, device):
        import torch
        qr, kr, ty = _host_slices(q_ranges, k_ranges, attn_type_map)
        stream = torch.cuda.current_stream(device).cuda_stream
        key = (device.index, stream, int(Tq), int(Tk), qr.tobytes(), kr.tobytes(), ty.tobytes())
        with self._lock:
            plan = self._plans.get(key)
            if plan is not None:
                self._plans.move_to_end(key)
                self.hits += 1
                return plan
        plan = ffa_plan_create(Tq, Tk, qr, kr, ty, device=device)
        evicted = []
        with self._lock:
            self.misses += 1
            self._plans[key] = plan
            while len(self._plans) > self.capacity:
                evicted.append(self._plans.popitem(last=False))
        for (dev_index, st, *_), old in evicted:
            _check(load_library().ffa_plan_destroy(old, st))
        return plan

    def clear(self):
        with self._lock:
            items = list(self._plans.items())
            self._plans.clear()
        for (dev_index, st, *_), old in items:
            _check(load_library().ffa_plan_destroy(old, st))


_PLAN_CACHE = _PlanCache(int(os.environ.get("FFA_PLAN_CACHE", "16")))


def cached_plan(Tq: int, Tk: int, q_ranges, k_ranges, attn_type_map, device=None):
    """A plan for these slices from the process-wide cache (``FFA_PLAN_CACHE``
    plans, default 16; 0 turns the cache off and returns None), made with
    ``ffa_plan_create`` on the current stream of ``device`` when not cached.
    The cache owns the plan: do not destroy it."""
    import torch
    if _PLAN_CACHE.capacity <= 0:
        return None
    dev_ = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    return _PLAN_CACHE.get(Tq, Tk, q_ranges, k_ranges, attn_type_map, dev_)


def clear_plan_cache() -> None:
    """Destroy every cached plan (stream-ordered on the streams they were made for)."""
    _PLAN_CACHE.clear()


FFA_PLAN_BAD_SLICE = 1
FFA_PLAN_CAPACITY = 2


def _cur_stream(device=None) -> int:
    import torch
    dev_ = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    return torch.cuda.current_stream(dev_).cuda_stream


def ffa_plan_device_workspace_size(Tq: int, Tk: int, R: int, max_entries: int) -> int:
    """C ABI ``ffa_plan_device_workspace_size``: bytes of workspace a device-built plan needs."""
    n = ctypes.c_size_t(0)
    _check(load_library().ffa_plan_device_workspace_size(Tq, Tk, R, max_entries, ctypes.byref(n)))
    return int(n.value)


def default_plan_capacity(Tq: int, Tk: int, R: int) -> int:
    """A generous entry capacity for device-built plans: every (row tile, key
    tile) pair of the 128 x 64 grid met by up to min(R, 16) slices."""
    return int(min((1 << 30) - 1, -(-Tq // 128) * -(-Tk // 64) * max(1, min(R, 16))))


def ffa_plan_create_device(Tq: int, Tk: int, q_ranges, k_ranges, attn_type_map,
                           max_entries: Optional[int] = None, workspace=None):
    """C ABI ``ffa_plan_create_device`` on device int32 tensors ([R,2], [R,2], [R]).

    Returns ``(plan, workspace)``; the workspace (allocated here if None) and
    the three slice tensors must stay alive, unmoved, until ffa_plan_destroy.
    """
    import torch
    for nm, t, nd in (("q_ranges", q_ranges, 2), ("k_ranges", k_ranges, 2), ("attn_type_map", attn_type_map, 1)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or t.dim() != nd \
                or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous int32 GPU tensor with {nd} dims")
    R = attn_type_map.shape[0]
    if tuple(q_ranges.shape) != (R, 2) or tuple(k_ranges.shape) != (R, 2):
        raise ValueError("q_ranges and k_ranges must be [R, 2] with attn_type_map [R]")
    if max_entries is None:
        max_entries = default_plan_capacity(Tq, Tk, R)
    need = ffa_plan_device_workspace_size(Tq, Tk, R, max_entries)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_ranges.device)
    h = ctypes.c_void_p()
    _check(load_library().ffa_plan_create_device(
        Tq, Tk, q_ranges.data_ptr(), k_ranges.data_ptr(), attn_type_map.data_ptr(), R, max_entries,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _cur_stream(q_ranges.device), ctypes.byref(h)))
    return h.value, workspace


def ffa_plan_refresh(plan, device=None) -> None:
    """C ABI ``ffa_plan_refresh`` on the current stream (capturable)."""
    _check(load_library().ffa_plan_refresh(plan, _cur_stream(device)))


def ffa_plan_status(plan, device=None) -> int:
    """C ABI ``ffa_plan_status``: FFA_PLAN_* bits of the last device build (synchronises)."""
    st = ctypes.c_int(0)
    _check(load_library().ffa_plan_status(plan, _cur_stream(device), ctypes.byref(st)))
    return int(st.value)


def ffa_plan_export(plan, which: int, device=None):
    """C ABI ``ffa_plan_export``: (row_ptr, entries [E,3], order) of list `which`
    (0 forward, 1 key-side dK/dV, 2 dQ), as ffa_plan_host returns them."""
    lib = load_library()
    s = _cur_stream(device)
    nt = ctypes.c_int64(0)
    n = lib.ffa_plan_export(plan, which, ctypes.byref(nt), None, None, 0, None, s)
    if n < 0:
        raise FfaError(int(n), ffa_last_error())
    row_ptr = np.zeros(nt.value + 1, dtype=np.int64)
    entries = np.zeros((max(n, 1), 3), dtype=np.int32)
    order = np.zeros(max(nt.value, 1), dtype=np.int32)
    n2 = lib.ffa_plan_export(plan, which, None, row_ptr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                             _iptr(entries), n, _iptr(order), s)
    if n2 != n:
        raise FfaError(int(n2), ffa_last_error())
    return row_ptr, entries[:n], order[:nt.value]


def ffa_fwd_planned(plan, q, k, v, scale: float, softcap: float = 0.0, out=None, lse=None,
                    alibi_slopes=None, saved=None, train: bool = False):
    """C ABI ``ffa_fwd_planned`` (``_ex`` with ``alibi_slopes`` or a saved record): the
    forward kernels alone.  Returns (out, lse), plus the record as in ``ffa_fwd``."""
    import torch
    lib = load_library()
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(nm, t, torch.bfloat16, 3)
    Tq, hq, d = q.shape
    hkv = k.shape[1]
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((Tq, hq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor("out", out, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    saved = _saved_tensor(saved, train, q, k)
    sp = _slopes_ptr(alibi_slopes, hq, q.device)
    head = (plan, q.data_ptr(), k.data_ptr(), v.data_ptr(), hq, hkv, d, float(scale), float(softcap))
    st = _stream_handle(q)
    if sp is None and saved is None:
        _check(lib.ffa_fwd_planned(*head, out.data_ptr(), lse.data_ptr(), st))
    else:
        _check(lib.ffa_fwd_planned_ex(*head, sp, out.data_ptr(), lse.data_ptr(),
                                      saved.data_ptr() if saved is not None else None, st))
    return (out, lse) if saved is None else (out, lse, saved)


def ffa_bwd_planned(plan, q, k, v, out, lse, dout, scale: float, softcap: float = 0.0,
                    dq=None, dk=None, dv=None, workspace=None, alibi_slopes=None, saved=None):
    """C ABI ``ffa_bwd_planned`` (``_ex`` with ``alibi_slopes`` or ``saved``): the
    backward kernels alone (plus a training-forward re-run when ``saved`` is None)."""
    import torch
    lib = load_library()
    for nm, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_tensor(nm, t, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    Tq, hq, d = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    ws_bytes = ffa_bwd_workspace_size(Tq, Tk, hq, hkv, d)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    saved = _saved_tensor(saved, False, q, k)
    sp = _slopes_ptr(alibi_slopes, hq, q.device)
    qkv = (plan, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    sizes = (hq, hkv, d, float(scale), float(softcap))
    tail = (dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_len, _stream_handle(q))
    if sp is None and saved is None:
        _check(lib.ffa_bwd_planned(*qkv, dout.data_ptr(), *sizes, *tail))
    else:
        _check(lib.ffa_bwd_planned_ex(*qkv, saved.data_ptr() if saved is not None else None,
                                      dout.data_ptr(), *sizes, sp, *tail))
    return dq, dk, dv


def ffa_fwd_ex(q, k, v, q_ranges, k_ranges, attn_type_map, scale: float, softcap: float,
               alibi_slopes, out=None, lse=None, saved=None, train: bool = False):
    """C ABI ``ffa_fwd_ex``: ``ffa_fwd`` with a distance bias (``alibi_slopes``: fp32 [hq] or None)
    and the optional saved record."""
    return ffa_fwd(q, k, v, q_ranges, k_ranges, attn_type_map, scale, softcap, out=out, lse=lse,
                   alibi_slopes=alibi_slopes, saved=saved, train=train)


def ffa_bwd_ex(q, k, v, out, lse, dout, q_ranges, k_ranges, attn_type_map, scale: float,
               softcap: float, alibi_slopes, dq=None, dk=None, dv=None, workspace=None, saved=None):
    """C ABI ``ffa_bwd_ex``: ``ffa_bwd`` with a distance bias (``alibi_slopes``: fp32 [hq] or None)
    and the training forward's ``saved`` record."""
    return ffa_bwd(q, k, v, out, lse, dout, q_ranges, k_ranges, attn_type_map, scale, softcap,
                   dq=dq, dk=dk, dv=dv, workspace=workspace, alibi_slopes=alibi_slopes, saved=saved)


def ffa_fwd_planned_ex(plan, q, k, v, scale: float, softcap: float, alibi_slopes, out=None, lse=None,
                       saved=None, train: bool = False):
    """C ABI ``ffa_fwd_planned_ex``: ``ffa_fwd_planned`` with a distance bias and the saved record."""
    return ffa_fwd_planned(plan, q, k, v, scale, softcap, out=out, lse=lse, alibi_slopes=alibi_slopes,
                           saved=saved, train=train)


def ffa_bwd_planned_ex(plan, q, k, v, out, lse, dout, scale: float, softcap: float, alibi_slopes,
                       dq=None, dk=None, dv=None, workspace=None, saved=None):
    """C ABI ``ffa_bwd_planned_ex``: ``ffa_bwd_planned`` with a distance bias and the saved record."""
    return ffa_bwd_planned(plan, q, k, v, out, lse, dout, scale, softcap, dq=dq, dk=dk, dv=dv,
                           workspace=workspace, alibi_slopes=alibi_slopes, saved=saved)


def flex_flash_attn_func(q, k, v, q_ranges, k_ranges, attn_type_map,
                         max_seqlen_q: Optional[int] = None, max_seqlen_k: Optional[int] = None,
                         softmax_scale: Optional[float] = None, softcap: float = 0.0,
                         alibi_slopes=None):
    """Range-masked attention with autograd.  Returns (out, lse); lse carries no gradient.

    ``alibi_slopes`` (fp32 [hq] on the GPU, or None) adds ``slope[h] * (j - i)``
    to every score after the softcap (``alibi_geometric_slopes(hq)`` gives ALiBi's
    geometric slopes); the slopes carry no gradient.

    Runs through the ``ffa_amd::fwd`` / ``ffa_amd::bwd`` custom operators
    (``torch_op``), so it also works inside ``torch.compile``: pad the slice
    lists with empty ``[x, x]`` slices to a fixed count and one compiled graph
    serves them all.  ``max_seqlen_q`` / ``max_seqlen_k`` are accepted for call
    compatibility and unused: the host planner derives the tiling from the
    ranges themselves.  Slice tensors on the GPU are copied to the host inside
    the operator (one synchronisation).
    """
    import torch

    def as_tensor(x):
        return x if isinstance(x, torch.Tensor) else torch.as_tensor(np.asarray(x, dtype=np.int32))

    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(q.shape[-1])
    # the training forward (which saves a record for the backward) when a
    # backward may follow
    train = torch.is_grad_enabled() and any(t.requires_grad for t in (q, k, v))
    out, lse, _ = torch.ops.ffa_amd.fwd(q, k, v, as_tensor(q_ranges), as_tensor(k_ranges),
                                        as_tensor(attn_type_map), float(softmax_scale), float(softcap),
                                        alibi_slopes, train)
    return out, lse


# Register the custom operators (ffa_amd::fwd, ffa_amd::bwd) on import, so
# compiled code never has to import anything.
try:
    from . import torch_op  # noqa: F401,E402
except ImportError:  # torch missing: the ctypes-level functions still work
    pass
