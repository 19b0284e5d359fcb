"""The custom operators under torch.compile, on the GPU.

The use case of the MagiAttention issue on dummy/padded attention slices:
pad the slice lists with empty slices to a fixed count so that torch.compile
sees static shapes.  Checked here:
  * the compiled function (fullgraph, aot_eager backend: the operators stay
    opaque, forward and backward graphs are traced through their fake
    implementations) gives bitwise the eager results, forward and gradients;
  * the eager results are bitwise those of the plain C ABI calls, which the
    parity tests compare with the oracle;
  * slice lists of the same padded length reuse one compiled graph.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, ffa, say

pytestmark = pytest.mark.gpu


def _attn(q, k, v, qr, kr, ty):
    out, lse = ffa.flex_flash_attn_func(q, k, v, qr, kr, ty, softmax_scale=None, softcap=0.0)
    return out, lse


def _slices_tensor(qr, kr, ty, d):
    return (torch.as_tensor(qr, dtype=torch.int32, device=d), torch.as_tensor(kr, dtype=torch.int32, device=d),
            torch.as_tensor(ty, dtype=torch.int32, device=d))


def _run(fn, q, k, v, do, sl, d):
    qd, kd, vd = (t.to(d).clone().requires_grad_() for t in (q, k, v))
    out, lse = fn(qd, kd, vd, *sl)
    out.backward(do.to(d))
    torch.cuda.synchronize()
    return out.detach(), lse.detach(), qd.grad, kd.grad, vd.grad


def test_eager_operator_matches_c_abi():
    w = W.config(2)
    say("eager custom operator vs C ABI (config 2)")
    q, k, v, do = W.workload_tensors(w, with_dout=True)
    d = dev()
    qr, kr, ty = w.slices()
    got = _run(_attn, q, k, v, do, _slices_tensor(qr, kr, ty, d), d)
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    # gradients are wanted, so the operator runs the training forward
    out, lse, rec = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, 0.0, train=True)
    dq, dk, dv = ffa.ffa_bwd(qd, kd, vd, out, lse, od, qr, kr, ty, w.scale, 0.0, saved=rec)
    torch.cuda.synchronize()
    for a, b in zip(got, (out, lse, dq, dk, dv)):
        assert torch.equal(a, b)


def test_compiled_matches_eager_and_reuses_graph():
    w = W.config(2)
    say("torch.compile fullgraph (aot_eager) vs eager, padded slices")
    q, k, v, do = W.workload_tensors(w, with_dout=True)
    d = dev()
    n_graphs = {"n": 0}
    inner = torch._dynamo.lookup_backend("aot_eager")

    def counting(gm, example_inputs):
        n_graphs["n"] += 1
        return inner(gm, example_inputs)

    torch._dynamo.reset()
    compiled = torch.compile(_attn, backend=counting, fullgraph=True)
    rng = np.random.default_rng(11)
    r_max = 24
    for trial in range(3):
        if trial == 0:
            qr, kr, ty = w.slices()
            qr, kr, ty = W.pad_slices(qr, kr, ty, r_max)
        else:
            qr, kr, ty = W.random_slices(rng, w.Tq, w.Tk, max_slices=8, n_dummies=0)
            qr, kr, ty = W.pad_slices(qr, kr, ty, r_max)
        sl = _slices_tensor(qr, kr, ty, d)
        eager = _run(_attn, q, k, v, do, sl, d)
        comp = _run(compiled, q, k, v, do, sl, d)
        for name, a, b in zip(("out", "lse", "dq", "dk", "dv"), comp, eager):
            assert torch.equal(a, b), (trial, name)
    # one graph for the three slice lists of the same padded length (the
    # compiled callable is a single graph; counting sees it once)
    assert n_graphs["n"] == 1, n_graphs
