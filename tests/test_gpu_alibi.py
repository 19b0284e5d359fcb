"""Distance bias (ALiBi) on the GPU: the biased kernels against the fp64 oracle.

The bias is slope[h] * (j - i) on every score after the softcap (the oracle's
reading of ALiBi as a distance-based bias).  Small problems are compared over
every element; the 64K-token batch and the mixed sink/window workload on
sampled rows and keys, as in the unbiased tests.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import O, check_grad, compare_out_lse, dev, ffa, say, to64

pytestmark = pytest.mark.gpu


def _slopes(rng, hq, kind):
    if kind == "alibi":
        return np.array(ffa.alibi_geometric_slopes(hq))
    return rng.uniform(-0.3, 0.3, hq)  # mixed signs: keys after the row gain, others lose


def _cmp(name, got, ref, ctx, mag):
    return check_grad(name, got, ref, ctx, mag)


CASES = [
    # (Tq, Tk, hq, hkv, d, softcap, seed, slope kind)
    (300, 300, 2, 1, 64, 0.0, 0, "alibi"),
    (257, 190, 4, 2, 128, 0.0, 1, "mixed"),
    (520, 700, 4, 4, 128, 30.0, 2, "mixed"),
    (129, 65, 8, 1, 64, 5.0, 3, "alibi"),
    (3, 700, 2, 1, 64, 0.0, 7, "mixed"),
]
IDS = [f"T{c[0]}x{c[1]}_h{c[2]}:{c[3]}_d{c[4]}_cap{c[5]}_{c[7]}" for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_slices_fwd_bwd_full_compare(case):
    Tq, Tk, hq, hkv, d, cap, seed, kind = case
    say(f"alibi fwd+bwd random slices {case}")
    rng = np.random.default_rng(seed + 300)
    dv_ = dev()
    for trial in range(2):
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=2)
        q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, d, seed=seed * 10 + trial)
        scale = float(rng.uniform(0.05, 0.3))
        sl = _slopes(rng, hq, kind)
        st = torch.tensor(sl, dtype=torch.float32, device=dv_)
        qd, kd, vd, od = q.to(dv_), k.to(dv_), v.to(dv_), do.to(dv_)
        out, lse = ffa.ffa_fwd_ex(qd, kd, vd, qr, kr, ty, scale, cap, st)
        dq, dk, dv = ffa.ffa_bwd_ex(qd, kd, vd, out, lse, od, qr, kr, ty, scale, cap, st)
        torch.cuda.synchronize()
        # the oracle sees the slopes the kernels saw (rounded to fp32)
        sl32 = st.double().cpu().numpy()
        ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, scale, cap,
                                           alibi_slopes=sl32)
        compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, f"{case} trial {trial}")
        rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, scale, cap,
                                           magnitudes=True, alibi_slopes=sl32)
        for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags):
            _cmp(n, g, r, f"{case} trial {trial}", m)


@pytest.mark.parametrize("cap", [0.0, 20.0])
def test_zero_slopes_forward_is_unbiased(cap):
    """With every slope 0 the biased forward adds exact zeros: without a
    softcap, the same bits.  With one, the unbiased forward folds the capped
    score cap - 2 cap r into its exp2 argument while the biased one rounds
    the capped score first, so the exp2 arguments (|arg| <= 2 cap log2 e,
    about 58 here) differ by a few fp32 ulps, 2^-18 each: each weight by a
    relative 2^-16 at most, which can move its fp16 rounding (for P V) by
    one fp16 ulp, 2^-10 of it.  The weights sum to l, so out moves by at
    most 2^-10 max|v| before its bf16 rounding and one bf16 ulp after it;
    lse by far less than 1e-4."""
    say(f"alibi zero slopes forward, softcap {cap}")
    w = W.config(2)
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    d = dev()
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    qr, kr, ty = w.slices()
    z = torch.zeros(w.hq, dtype=torch.float32, device=d)
    o0, l0 = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, cap)
    o1, l1 = ffa.ffa_fwd_ex(qd, kd, vd, qr, kr, ty, w.scale, cap, z)
    torch.cuda.synchronize()
    if cap == 0.0:
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        return
    o0, o1 = o0.float(), o1.float()
    ulp = torch.exp2(torch.floor(torch.log2(torch.maximum(o0.abs(), o1.abs()).clamp_min(2.0 ** -100))) - 7)
    diff = (o0 - o1).abs()
    say(f"  out max diff {diff.max().item():.3g}, lse max diff {(l0 - l1).abs().max().item():.3g}")
    assert (diff <= 2.0 ** -10 * vd.float().abs().max() + ulp).all()
    assert (l0 - l1).abs().max().item() < 1e-4


@pytest.mark.parametrize("n", [4, 5])
def test_full_size_sampled(n):
    """ALiBi's geometric slopes on the 64K-token batch and on the mixed
    sink/window workload (softcap 50): sampled rows of out, lse and dq, and
    keys near a document's end for dk, dv."""
    w = W.config(n)
    say(f"alibi full size config {n} ({w.name})")
    q, k, v, do = W.workload_tensors(w)
    qr, kr, ty = w.slices()
    d = dev()
    st = torch.tensor(ffa.alibi_geometric_slopes(w.hq), dtype=torch.float32, device=d)
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    out, lse = ffa.ffa_fwd_ex(qd, kd, vd, qr, kr, ty, w.scale, w.softcap, st)
    dq, dk, dv = ffa.ffa_bwd_ex(qd, kd, vd, out, lse, od, qr, kr, ty, w.scale, w.softcap, st)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    sl32 = st.double().cpu().numpy()
    rng = np.random.default_rng(n + 70)
    e0 = 8192 * 7 if n == 4 else w.Tk
    rows = np.unique(np.concatenate([rng.integers(e0 - 1024, e0, 24), [e0 - 1024, e0 - 897, e0 - 1]]))
    keys = np.array([e0 - 130, e0 - 65, e0 - 64, e0 - 2, e0 - 1])
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, w.scale, w.softcap,
                                       rows=rows, alibi_slopes=sl32)
    e_out, e_lse = compare_out_lse(out[rows].cpu(), lse[rows].cpu(), ref_out, ref_lse, f"config {n}")
    rq, rk, rv, (mq, mk, mv) = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, w.scale,
                                               w.softcap, rows=rows, keys=keys, magnitudes=True,
                                               alibi_slopes=sl32)
    e = [_cmp("dq", dq[rows], rq, f"config {n}", mq), _cmp("dk", dk[keys], rk, f"config {n}", mk),
         _cmp("dv", dv[keys], rv, f"config {n}", mv)]
    say(f"  out {e_out:.3e} lse {e_lse:.3e} dq/dk/dv {e[0]:.3e} {e[1]:.3e} {e[2]:.3e}")


def test_planned_and_autograd_paths():
    """The planned entry points and flex_flash_attn_func (which runs the
    training forward when gradients are wanted) give the one-shot bits."""
    w = W.config(1)
    say("alibi planned + autograd")
    q, k, v, do = W.workload_tensors(w, with_dout=True)
    d = dev()
    qr, kr, ty = w.slices()
    st = torch.tensor([0.5, -0.25], dtype=torch.float32, device=d)
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    o0, l0, r0 = ffa.ffa_fwd_ex(qd, kd, vd, qr, kr, ty, w.scale, 0.0, st, train=True)
    g0 = ffa.ffa_bwd_ex(qd, kd, vd, o0, l0, od, qr, kr, ty, w.scale, 0.0, st, saved=r0)
    plan = ffa.ffa_plan_create(w.Tq, w.Tk, qr, kr, ty)
    try:
        o1, l1, r1 = ffa.ffa_fwd_planned_ex(plan, qd, kd, vd, w.scale, 0.0, st, train=True)
        g1 = ffa.ffa_bwd_planned_ex(plan, qd, kd, vd, o1, l1, od, w.scale, 0.0, st, saved=r1)
    finally:
        ffa.ffa_plan_destroy(plan)
    qa, ka, va = (t.clone().requires_grad_() for t in (qd, kd, vd))
    o2, l2 = ffa.flex_flash_attn_func(qa, ka, va, qr, kr, ty, softmax_scale=w.scale, alibi_slopes=st)
    o2.backward(od)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1) and torch.equal(o0, o2) and torch.equal(l0, l2)
    for a, b, c in zip(g0, g1, (qa.grad, ka.grad, va.grad)):
        assert torch.equal(a, b) and torch.equal(a, c)
