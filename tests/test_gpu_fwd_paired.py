"""The forward with two q heads per workgroup.

Where q heads pair up within a kv head, large grids run the forward with two
q heads of one kv head per workgroup (eight waves sharing every K and V tile
in LDS).  Per row it does the same arithmetic in the same order as with one
head per workgroup, so the two must agree bitwise; both are also compared with
the fp64 oracle.  FFA_FWD_PAIRED forces the choice (by default the grid size
makes it, and the small cases here would run one head per workgroup).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import O, compare_out_lse, dev, ffa, say, to64

pytestmark = pytest.mark.gpu


def _fwd(monkeypatch, paired, q, k, v, qr, kr, ty, scale, cap, train=False):
    monkeypatch.setenv("FFA_FWD_PAIRED", "1" if paired else "0")
    r = ffa.ffa_fwd(q, k, v, qr, kr, ty, scale, cap, train=train)
    torch.cuda.synchronize()
    return r


CASES = [
    # (Tq, Tk, hq, hkv, d, softcap, seed): ragged tails, group sizes 2..8, both head sizes
    (300, 300, 2, 1, 64, 0.0, 0),
    (257, 190, 4, 2, 128, 0.0, 1),
    (520, 700, 8, 2, 128, 30.0, 2),
    (129, 65, 8, 1, 64, 5.0, 3),
    (1000, 1000, 4, 2, 128, 0.0, 4),
    (64, 64, 2, 1, 64, 0.0, 5),
    (1, 1, 2, 1, 128, 0.0, 6),
    (3, 700, 2, 1, 64, 0.0, 7),
    (777, 1500, 16, 2, 128, 50.0, 8),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}x{c[1]}_h{c[2]}:{c[3]}_d{c[4]}_cap{c[5]}" for c in CASES])
def test_paired_matches_one_head_and_oracle(case, monkeypatch):
    Tq, Tk, hq, hkv, d, cap, seed = case
    say(f"fwd two heads per workgroup {case}")
    rng = np.random.default_rng(100 + seed)
    dv_ = dev()
    for trial in range(3):
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=2)
        q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=seed * 10 + trial, with_dout=False)
        scale = float(rng.uniform(0.05, 0.3))
        qd, kd, vd = q.to(dv_), k.to(dv_), v.to(dv_)
        o1, l1 = _fwd(monkeypatch, True, qd, kd, vd, qr, kr, ty, scale, cap)
        o0, l0 = _fwd(monkeypatch, False, qd, kd, vd, qr, kr, ty, scale, cap)
        assert torch.equal(o1, o0), f"{case} trial {trial}: out differs from one head per workgroup"
        assert torch.equal(l1, l0), f"{case} trial {trial}: lse differs from one head per workgroup"
        ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, scale, cap)
        compare_out_lse(o1.cpu(), l1.cpu(), ref_out, ref_lse, f"{case} trial {trial}")


@pytest.mark.parametrize("n", [2, 1])
def test_paired_configs_and_training_record(n, monkeypatch):
    """Configurations with group sizes 4 and 2, plain and training forward:
    bitwise equal to one head per workgroup (out, lse and the record's
    defined bytes), and the plain output against the oracle."""
    w = W.config(n)
    say(f"fwd two heads per workgroup, config {n} ({w.name})")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    qr, kr, ty = w.slices()
    dv_ = dev()
    qd, kd, vd = q.to(dv_), k.to(dv_), v.to(dv_)
    o1, l1 = _fwd(monkeypatch, True, qd, kd, vd, qr, kr, ty, w.scale, w.softcap)
    o0, l0 = _fwd(monkeypatch, False, qd, kd, vd, qr, kr, ty, w.scale, w.softcap)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    t1 = _fwd(monkeypatch, True, qd, kd, vd, qr, kr, ty, w.scale, w.softcap, train=True)
    t0 = _fwd(monkeypatch, False, qd, kd, vd, qr, kr, ty, w.scale, w.softcap, train=True)
    assert torch.equal(t1[0], t0[0]) and torch.equal(t1[1], t0[1])
    # the record's defined bytes: the range words, out's residual, v's fp16
    # copy (padding between them is never written)
    n_out, n_v = 2 * q.numel(), 2 * k.numel()
    v16 = 256 + (n_out + 255) // 256 * 256
    for lo, hi in ((0, 16), (256, 256 + n_out), (v16, v16 + n_v)):
        assert torch.equal(t1[2][lo:hi], t0[2][lo:hi]), f"record bytes {lo}..{hi}"

    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, w.scale, w.softcap)
    compare_out_lse(o1.cpu(), l1.cpu(), ref_out, ref_lse, f"config {n}")


def test_paired_split_q_tiles(monkeypatch):
    """A long context against few q rows: the list is cut into runs, each run
    a two-head workgroup, merged by fwd_combine."""
    say("fwd two heads per workgroup, split q tiles")
    Tq, Tk, hq, hkv, d = 200, 40000, 4, 2, 128
    qr, kr, ty = [[0, Tq], [7, 7]], [[0, Tk], [0, 0]], [0, 0]
    q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=31, with_dout=False)
    dv_ = dev()
    qd, kd, vd = q.to(dv_), k.to(dv_), v.to(dv_)
    o1, l1 = _fwd(monkeypatch, True, qd, kd, vd, qr, kr, ty, d ** -0.5, 0.0)
    o0, l0 = _fwd(monkeypatch, False, qd, kd, vd, qr, kr, ty, d ** -0.5, 0.0)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, d ** -0.5, 0.0)
    compare_out_lse(o1.cpu(), l1.cpu(), ref_out, ref_lse, "split")


def test_paired_distance_bias(monkeypatch):
    """ALiBi with geometric (positive) slopes: every head walks its list from
    the last key tile down, with two heads per workgroup as with one."""
    say("fwd two heads per workgroup, distance bias")
    Tq, Tk, hq, hkv, d = 700, 900, 8, 2, 128
    rng = np.random.default_rng(41)
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=2)
    q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=41, with_dout=False)
    slopes = np.array(ffa.alibi_geometric_slopes(hq))
    dv_ = dev()
    st = torch.tensor(slopes, dtype=torch.float32, device=dv_)
    qd, kd, vd = q.to(dv_), k.to(dv_), v.to(dv_)
    outs = []
    for paired in (True, False):
        monkeypatch.setenv("FFA_FWD_PAIRED", "1" if paired else "0")
        outs.append(ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, d ** -0.5, 0.0, alibi_slopes=st))
        torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, d ** -0.5, 0.0,
                                       alibi_slopes=slopes)
    compare_out_lse(outs[0][0].cpu(), outs[0][1].cpu(), ref_out, ref_lse, "alibi")
