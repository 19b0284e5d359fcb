"""The C ABI: the library loads, exports what include/ffa.h declares, and
rejects bad arguments before any GPU work (so these run without a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

from _lib import ROOT, ensure_built, ffa


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def _declared():
    src = open(os.path.join(ROOT, "include", "ffa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ffa_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"ffa_fwd", "ffa_bwd", "ffa_bwd_workspace_size", "ffa_plan_host",
            "ffa_last_error", "ffa_build_info", "ffa_plan_create", "ffa_fwd_planned",
            "ffa_bwd_planned", "ffa_plan_destroy"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    # the python binding carries the same names
    for n in names:
        assert hasattr(ffa, n), n


def test_build_info(lib):
    info = ffa.ffa_build_info()
    assert "arch=gfx950" in info
    # the library was built from the sources in this tree (a stale build
    # would carry another hash: rebuild with __graft_entry__.build())
    from range_masked_attention_amd import _build
    assert f"source={_build.source_hash()}" in info, info
    # every tile shape the planner is asked for is reported
    for key in ("fwd_tile=", "bwd_kv_tile=", "bwd_q_tile="):
        assert key in info, info


def _fwd(lib, Tq=16, Tk=16, hq=2, hkv=1, d=64, qr=((0, 16),), kr=((0, 16),), ty=(0,),
         scale=0.125, softcap=0.0, ptr=64):
    qr = np.ascontiguousarray(np.asarray(qr, np.int32).reshape(-1, 2))
    kr = np.ascontiguousarray(np.asarray(kr, np.int32).reshape(-1, 2))
    ty = np.ascontiguousarray(np.asarray(ty, np.int32).reshape(-1))
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    # pointers are never dereferenced: every case fails validation (or Tq == 0)
    return lib.ffa_fwd(ptr, ptr, ptr, Tq, Tk, hq, hkv, d, ip(qr), ip(kr), ip(ty), qr.shape[0],
                       scale, softcap, ptr, ptr, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(hq=3, hkv=2), -1, "multiple"),
    (dict(hkv=0), -1, "positive"),
    (dict(d=96), -2, "96"),
    (dict(scale=0.0), -1, "scale"),
    (dict(scale=float("nan")), -1, "scale"),
    (dict(softcap=-1.0), -1, "softcap"),
    (dict(softcap=float("inf")), -1, "softcap"),
    (dict(qr=((5, 3),)), -1, "q range"),
    (dict(kr=((0, 17),)), -1, "k range"),
    (dict(qr=((-1, 3),)), -1, "q range"),
    (dict(ty=(2,)), -1, "type"),
    (dict(Tq=-1), -1, ">= 0"),
    (dict(Tq=1 << 30, hq=2, d=64), -1, "2^31"),
])
def test_invalid_arguments(lib, kw, code, msg):
    rc = _fwd(lib, **kw)
    assert rc == code
    assert msg in ffa.ffa_last_error()


def test_null_pointers_rejected(lib):
    assert _fwd(lib, ptr=None) == -1
    assert "NULL" in ffa.ffa_last_error()


def test_empty_query_axis_is_a_no_op(lib):
    # nothing to compute: returns before any HIP call
    assert _fwd(lib, Tq=0, qr=((0, 0),)) == 0


def test_overlap_rejected_in_debug_mode(lib, monkeypatch):
    monkeypatch.setenv("FFA_DEBUG", "1")
    assert _fwd(lib, qr=((0, 16), (4, 8)), kr=((0, 16), (3, 5)), ty=(0, 1), ptr=None) == -1
    assert "same cells" in ffa.ffa_last_error()
    # disjoint slices (causal triangles that never meet) pass the debug check and then
    # fail only on the NULL pointers
    assert _fwd(lib, qr=((0, 8), (8, 16)), kr=((0, 8), (0, 16)), ty=(1, 1), ptr=None) == -1
    assert "NULL" in ffa.ffa_last_error()


def test_bwd_validation(lib):
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    qr = np.array([[0, 4]], np.int32); kr = np.array([[0, 9]], np.int32); ty = np.array([1], np.int32)
    rc = lib.ffa_bwd(64, 64, 64, 64, 64, 64, 4, 8, 2, 2, 64, ip(qr), ip(kr), ip(ty), 1,
                     0.1, 0.0, 64, 64, 64, None, 0, None)
    assert rc == -1 and "k range" in ffa.ffa_last_error()
    # workspace: D [Tq][hq] fp32; with keys, fp32 partial dK/dV of at most 512
    # (run, kv head) pairs of 128 keys x d x 2; with rows, fp32 partial dQ of
    # at most 512 (run, q head) pairs of 128 rows x d; fp16 copies of q, dO
    # (rows) and k (keys); the forward re-run's out and saved record (out's
    # residual, v's fp16 copy)
    dkv, dq = 512 * 2 * 128 * 4, 512 * 128 * 4  # per unit of d
    rows = 100 * 8 * 64 * 2 * 4  # q16, do16, out, residual at d = 64
    assert 100 * 8 * 4 + dq * 64 + rows <= lib.ffa_bwd_workspace_size(100, 0, 8, 2, 64) \
        < 100 * 8 * 4 + dq * 64 + rows + (1 << 20)
    keys = 256 * 2 * 64 * 2 * 2  # k16, the record's v16
    assert dkv * 64 + keys <= lib.ffa_bwd_workspace_size(0, 256, 8, 2, 64) < dkv * 64 + keys + (1 << 20)
    assert lib.ffa_bwd_workspace_size(100, 256, 8, 2, 128) >= 100 * 8 * 4 + (dkv + dq) * 128
    assert lib.ffa_bwd_workspace_size(100, 256, 8, 2, 64) < lib.ffa_bwd_workspace_size(100, 256, 8, 2, 128)
    assert lib.ffa_bwd_workspace_size(0, 0, 8, 2, 64) == 0
    assert lib.ffa_bwd_workspace_size(100, 256, 8, 2, 96) == 0
    assert lib.ffa_bwd_workspace_size(100, 256, 0, 2, 64) == 0


def test_plan_api_validation(lib):
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    qr = np.array([[0, 4]], np.int32); kr = np.array([[2, 1]], np.int32); ty = np.array([0], np.int32)
    h = ctypes.c_void_p()
    assert lib.ffa_plan_create(4, 8, ip(qr), ip(kr), ip(ty), 1, None, ctypes.byref(h)) == -1
    assert "k range" in ffa.ffa_last_error() and h.value is None
    assert lib.ffa_plan_create(4, 8, ip(qr), ip(kr), ip(ty), 1, None, None) == -1
    assert lib.ffa_fwd_planned(None, 64, 64, 64, 1, 1, 64, 0.1, 0.0, 64, 64, None) == -1
    assert "plan" in ffa.ffa_last_error()
    assert lib.ffa_plan_destroy(None, None) == 0


def test_misaligned_pointer_rejected(lib):
    assert _fwd(lib, ptr=72) == -1
    assert "aligned" in ffa.ffa_last_error()


def test_alibi_slopes_validation(lib):
    """A misaligned slope pointer is rejected before any GPU work."""
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    qr = np.array([[0, 4]], np.int32); kr = np.array([[0, 4]], np.int32); ty = np.array([1], np.int32)
    rc = lib.ffa_fwd_ex(64, 64, 64, 4, 4, 2, 2, 64, ip(qr), ip(kr), ip(ty), 1, 0.1, 0.0, 66, 64, 64, None,
                        None)
    assert rc == -1 and "alibi_slopes" in ffa.ffa_last_error()
    rc = lib.ffa_bwd_ex(64, 64, 64, 64, 64, None, 64, 4, 4, 2, 2, 64, ip(qr), ip(kr), ip(ty), 1,
                        0.1, 0.0, 66, 64, 64, 64, None, 0, None)
    assert rc == -1 and "alibi_slopes" in ffa.ffa_last_error()


def test_saved_record_validation(lib):
    """A misaligned saved-record pointer is rejected before any GPU work, and
    the record's size is its header plus 2 bytes per element of q and of v,
    plus the v copy pass's 2048 partial maxima."""
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    qr = np.array([[0, 4]], np.int32); kr = np.array([[0, 4]], np.int32); ty = np.array([1], np.int32)
    rc = lib.ffa_fwd_ex(64, 64, 64, 4, 4, 2, 2, 64, ip(qr), ip(kr), ip(ty), 1, 0.1, 0.0, None, 64, 64, 72,
                        None)
    assert rc == -1 and "saved" in ffa.ffa_last_error()
    rc = lib.ffa_bwd_ex(64, 64, 64, 64, 64, 72, 64, 4, 4, 2, 2, 64, ip(qr), ip(kr), ip(ty), 1,
                        0.1, 0.0, None, 64, 64, 64, None, 0, None)
    assert rc == -1 and "saved" in ffa.ffa_last_error()
    r256 = lambda x: (x + 255) // 256 * 256
    assert lib.ffa_saved_size(100, 300, 8, 2, 128) == \
        256 + r256(100 * 8 * 128 * 2) + r256(300 * 2 * 128 * 2) + 2048 * 4
    assert lib.ffa_saved_size(100, 300, 8, 2, 96) == 0


def test_noalloc_rejects_sizes_beyond_its_array(lib):
    """ffa_fwd_noalloc checks its limits on the host, before any GPU work:
    more than 4096 slices, or a plan larger than its device array."""
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    R = 4097
    qr = np.zeros((R, 2), np.int32); kr = np.zeros((R, 2), np.int32); ty = np.zeros(R, np.int32)
    rc = lib.ffa_fwd_noalloc(64, 64, 64, 16, 16, 2, 1, 64, ip(qr), ip(kr), ip(ty), R, 0.1, 0.0, 64, 64, None)
    assert rc == -1 and "4096 slices" in ffa.ffa_last_error()
    # one FULL slice over 2^20 x 2^20 tokens: 8192 x 16384 tiles, far past the array
    T = 1 << 20
    qr = np.array([[0, T]], np.int32); kr = np.array([[0, T]], np.int32); ty = np.array([0], np.int32)
    rc = lib.ffa_fwd_noalloc(64, 64, 64, T, T, 1, 1, 64, ip(qr), ip(kr), ip(ty), 1, 0.1, 0.0, 64, 64, None)
    assert rc == -1 and "entries" in ffa.ffa_last_error() and "134217728" in ffa.ffa_last_error()
    # v's fp16 copy alone past the array: 2^20 tokens x 2 kv heads x d 128 x 2 bytes = 512 MiB
    rc = lib.ffa_fwd_noalloc(64, 64, 64, T, T, 2, 2, 128, ip(qr), ip(kr), ip(ty), 1, 0.1, 0.0, 64, 64, None)
    assert rc == -1 and "fp16 copy of v" in ffa.ffa_last_error() and "268435456" in ffa.ffa_last_error()
    # bad slices are reported as by ffa_fwd
    qr = np.array([[0, 17]], np.int32); kr = np.array([[0, 16]], np.int32); ty = np.array([0], np.int32)
    rc = lib.ffa_fwd_noalloc(64, 64, 64, 16, 16, 2, 1, 64, ip(qr), ip(kr), ip(ty), 1, 0.1, 0.0, 64, 64, None)
    assert rc == -1 and "q range" in ffa.ffa_last_error()


def test_injected_host_allocation_failure(lib, monkeypatch):
    """FFA_INJECT_NOMEM makes every host planning step fail as if the host
    allocator had run out: the host-only entry points then return
    FFA_ERR_NOMEM (-4) with a message, and work again once it is unset."""
    qr, kr, ty = [[0, 300]], [[0, 300]], [1]
    monkeypatch.setenv("FFA_INJECT_NOMEM", "1")
    with pytest.raises(ffa.FfaError) as e:
        ffa.ffa_plan_host(300, 300, qr, kr, ty, 128, 64)
    assert e.value.code == -4 and "out of host memory" in str(e.value)
    with pytest.raises(ffa.FfaError) as e:
        ffa.ffa_block_slices([1, 2], [[0, 0], [0, 1]], 256, 256)
    assert e.value.code == -4 and "out of host memory" in str(e.value)
    # the plan handle entry point fails before any device work
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    q = np.array(qr, np.int32); k = np.array(kr, np.int32); t = np.array(ty, np.int32)
    h = ctypes.c_void_p()
    assert lib.ffa_plan_create(300, 300, ip(q), ip(k), ip(t), 1, None, ctypes.byref(h)) == -4
    assert h.value is None and "out of host memory" in ffa.ffa_last_error()
    monkeypatch.setenv("FFA_INJECT_NOMEM", "0")
    row_ptr, ent, order = ffa.ffa_plan_host(300, 300, qr, kr, ty, 128, 64)
    assert row_ptr[-1] == len(ent) > 0


def test_probe_library_exports_its_entry_point(lib):
    """The matrix-core rate probe bench.py --mfma-ceiling loads is a library
    of its own (nothing of it is in libffa.so) with one C entry point."""
    from range_masked_attention_amd import _build
    if not os.path.exists(_build.PROBE_LIB):
        _build.build_probe(_build._hipcc())
    probe = ctypes.CDLL(_build.PROBE_LIB)
    assert hasattr(probe, "ffa_probe_mfma_rate")
    assert not hasattr(lib, "ffa_probe_mfma_rate")
