"""Plans built on the device (ffa_plan_create_device) against the host planner.

Integer work, so the bar is exact: each of the three block lists (forward,
key-side dK/dV, dQ) read back with ffa_plan_export must equal ffa_plan_host's
list for the same tiling, entry for entry and in the same tile order, on
ragged random slice lists (with empty slices anywhere, any order) and on the
five workload configs.  The attention outputs with a device-built plan must
then be bitwise those with a host-built plan.  Also: the status bits, and a
captured HIP graph (refresh + forward + backward) replayed on new slice lists.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, ffa, say

pytestmark = pytest.mark.gpu

FWD = (128, 64, False)   # forward and dQ lists: q tiles of 128 rows, k tiles of 64
KV = (64, 128, True)     # dK/dV list: k tiles of 128 keys, q tiles of 64 rows


def _dev_slices(qr, kr, ty, d):
    return (torch.as_tensor(np.asarray(qr, dtype=np.int32), device=d).contiguous(),
            torch.as_tensor(np.asarray(kr, dtype=np.int32), device=d).contiguous(),
            torch.as_tensor(np.asarray(ty, dtype=np.int32), device=d).contiguous())


def _same(a, b):
    return all(np.array_equal(x, y) for x, y in zip(a, b))


def _check_lists(Tq, Tk, qr, kr, ty, d, ctx):
    sl = _dev_slices(qr, kr, ty, d)
    plan, ws = ffa.ffa_plan_create_device(Tq, Tk, *sl)
    hplan = ffa.ffa_plan_create(Tq, Tk, qr, kr, ty)
    try:
        assert ffa.ffa_plan_status(plan) == 0, ctx
        for which, tiling in ((0, FWD), (1, KV), (2, FWD)):
            ref = ffa.ffa_plan_host(Tq, Tk, qr, kr, ty, *tiling)
            got = ffa.ffa_plan_export(plan, which)
            assert _same(got, ref), f"{ctx}: device list {which} differs"
            assert _same(ffa.ffa_plan_export(hplan, which), ref), f"{ctx}: host plan export {which}"
    finally:
        ffa.ffa_plan_destroy(plan)
        ffa.ffa_plan_destroy(hplan)
        torch.cuda.synchronize()


def test_random_slices_exact():
    d = dev()
    rng = np.random.default_rng(2024)
    say("device planner: 80 random slice lists")
    for trial in range(80):
        Tq, Tk = int(rng.integers(1, 1500)), int(rng.integers(1, 1500))
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=10, n_dummies=int(rng.integers(0, 5)))
        perm = rng.permutation(len(ty))
        _check_lists(Tq, Tk, qr[perm], kr[perm], ty[perm], d, f"trial {trial} Tq={Tq} Tk={Tk}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_configs_exact(n):
    w = W.config(n)
    say(f"device planner: config {n}")
    qr, kr, ty = w.slices()
    _check_lists(w.Tq, w.Tk, qr, kr, ty, dev(), f"config {n}")


def test_attention_with_device_plan_is_bitwise_host_plan():
    w = W.config(5)
    say("attention with a device-built plan (config 5 slices, 4/1 heads)")
    d = dev()
    q, k, v, do = W.make_tensors(w.Tq, w.Tk, 4, 1, 128, seed=9)
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    qr, kr, ty = w.slices()
    plan, ws = ffa.ffa_plan_create_device(w.Tq, w.Tk, *_dev_slices(qr, kr, ty, d))
    hplan = ffa.ffa_plan_create(w.Tq, w.Tk, qr, kr, ty)
    try:
        o1, l1 = ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, w.softcap)
        g1 = ffa.ffa_bwd_planned(plan, qd, kd, vd, o1, l1, od, w.scale, w.softcap)
        o0, l0 = ffa.ffa_fwd_planned(hplan, qd, kd, vd, w.scale, w.softcap)
        g0 = ffa.ffa_bwd_planned(hplan, qd, kd, vd, o0, l0, od, w.scale, w.softcap)
        torch.cuda.synchronize()
    finally:
        ffa.ffa_plan_destroy(plan)
        ffa.ffa_plan_destroy(hplan)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    for x, y in zip(g1, g0):
        assert torch.equal(x, y)


def test_status_bad_slice_and_capacity():
    d = dev()
    say("device planner status: bad slice, capacity")
    Tq = Tk = 300
    q, k, v, _ = W.make_tensors(Tq, Tk, 2, 1, 64, seed=1)
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    # a slice past the end of the keys
    qr, kr, ty = np.array([[0, 300]]), np.array([[0, 301]]), np.array([1])
    plan, ws = ffa.ffa_plan_create_device(Tq, Tk, *_dev_slices(qr, kr, ty, d))
    try:
        assert ffa.ffa_plan_status(plan) & ffa.FFA_PLAN_BAD_SLICE
        out, lse = ffa.ffa_fwd_planned(plan, qd, kd, vd, 0.125, 0.0)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out) == 0 and bool(torch.all(torch.isneginf(lse)))
        assert ffa.ffa_plan_export(plan, 0)[1].shape[0] == 0
    finally:
        ffa.ffa_plan_destroy(plan)
    # a valid list that needs more entries than the capacity given
    qr, kr, ty = np.array([[0, 300]]), np.array([[0, 300]]), np.array([0])
    need = ffa.ffa_plan_host(Tq, Tk, qr, kr, ty, *FWD)[1].shape[0]
    plan, ws = ffa.ffa_plan_create_device(Tq, Tk, *_dev_slices(qr, kr, ty, d), max_entries=need - 1)
    try:
        assert ffa.ffa_plan_status(plan) & ffa.FFA_PLAN_CAPACITY
    finally:
        ffa.ffa_plan_destroy(plan)
    plan, ws = ffa.ffa_plan_create_device(Tq, Tk, *_dev_slices(qr, kr, ty, d), max_entries=need)
    try:
        assert ffa.ffa_plan_status(plan) == 0
    finally:
        ffa.ffa_plan_destroy(plan)
        torch.cuda.synchronize()


def test_graph_capture_replays_new_slice_lists():
    """refresh + training forward (into a saved record, which holds v's fp16
    copy, so that nothing is allocated under capture) + backward on that
    record, captured once and replayed on three slice lists copied into the
    same device arrays; every replay equals the eager one-shot calls
    bitwise, with eager work and synchronisation between."""
    w = W.config(2)
    say("HIP graph: refresh + fwd + bwd, replayed on new slice lists")
    d = dev()
    q, k, v, do = W.workload_tensors(w, with_dout=True)
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    r_max = 16
    rng = np.random.default_rng(5)
    lists = [W.pad_slices(*w.slices(padded=False), r_max)]
    for _ in range(2):
        lists.append(W.pad_slices(*W.random_slices(rng, w.Tq, w.Tk, max_slices=6, n_dummies=0), r_max))
    sq, sk, st = _dev_slices(*lists[0], d)
    plan, ws = ffa.ffa_plan_create_device(w.Tq, w.Tk, sq, sk, st)
    out = torch.empty_like(qd)
    lse = torch.empty((w.Tq, w.hq), dtype=torch.float32, device=d)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    bws = torch.empty(max(ffa.ffa_bwd_workspace_size(w.Tq, w.Tk, w.hq, w.hkv, w.d), 16), dtype=torch.uint8, device=d)
    rec = torch.empty(ffa.ffa_saved_size(w.Tq, w.Tk, w.hq, w.hkv, w.d), dtype=torch.uint8, device=d)

    def body():
        ffa.ffa_plan_refresh(plan)
        ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, 0.0, out=out, lse=lse, saved=rec)
        ffa.ffa_bwd_planned(plan, qd, kd, vd, out, lse, od, w.scale, 0.0, dq=dq, dk=dk, dv=dv,
                            workspace=bws, saved=rec)

    try:
        side = torch.cuda.Stream(device=d)
        side.wait_stream(torch.cuda.current_stream(d))
        with torch.cuda.stream(side):
            body()  # warm-up outside the capture
        torch.cuda.current_stream(d).wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        for rep in range(2):
            for i, (qr, kr, ty) in enumerate(lists):
                nq, nk, nt = _dev_slices(qr, kr, ty, d)
                sq.copy_(nq)
                sk.copy_(nk)
                st.copy_(nt)
                g.replay()
                torch.cuda.synchronize()
                assert ffa.ffa_plan_status(plan) == 0
                o0, l0 = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, 0.0)
                g0 = ffa.ffa_bwd(qd, kd, vd, o0, l0, od, qr, kr, ty, w.scale, 0.0)
                torch.cuda.synchronize()
                assert torch.equal(out, o0) and torch.equal(lse, l0), (rep, i)
                for x, y in zip((dq, dk, dv), g0):
                    assert torch.equal(x, y), (rep, i)
        del g
    finally:
        torch.cuda.synchronize()
        ffa.ffa_plan_destroy(plan)
