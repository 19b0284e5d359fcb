"""ffa_fwd_noalloc (through the C ABI) against ffa_fwd: the same bits, with
the plan and run scratch in the library's own device array.

Two calls in a row on different inputs, the second smaller, so the second
must not see anything of the first; a long-context case whose q-tile lists
are cut into runs (the run scratch in the array); and a call that leaves a
row with nothing visible.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, ffa, say

pytestmark = pytest.mark.gpu


def _both(q, k, v, qr, kr, ty, scale, cap, d):
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    out = torch.full_like(qd, 3.0)
    lse = torch.full((q.shape[0], q.shape[1]), 3.0, dtype=torch.float32, device=d)
    ffa.ffa_fwd_noalloc(qd, kd, vd, qr, kr, ty, scale, cap, out, lse)
    ref_out, ref_lse = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, cap)
    torch.cuda.synchronize()
    return out, lse, ref_out, ref_lse


def test_noalloc_matches_ffa_fwd_twice_then_smaller():
    d = dev()
    cases = []
    w = W.config(2)
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    cases.append(("config 2", q, k, v, *w.slices(), w.scale, 0.0))
    w = W.config(1)
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    cases.append(("config 1 (smaller)", q, k, v, *w.slices(), w.scale, 0.0))
    # short query block against a long context: lists cut into runs
    q, k, v, _ = W.make_tensors(256, 32768, 4, 1, 128, seed=21, with_dout=False)
    cases.append(("long context", q, k, v, np.array([[0, 256]], np.int32), np.array([[0, 32768]], np.int32),
                  np.array([0], np.int32), 128 ** -0.5, 0.0))
    # softcap, rows 0..99 see nothing
    q, k, v, _ = W.make_tensors(300, 100, 2, 1, 64, seed=11, with_dout=False)
    cases.append(("causal Lk < Lq, softcap", q, k, v, np.array([[0, 300]], np.int32),
                  np.array([[0, 100]], np.int32), np.array([1], np.int32), 0.1, 5.0))
    for name, q, k, v, qr, kr, ty, scale, cap in cases:
        say(f"noalloc vs ffa_fwd: {name}")
        out, lse, ref_out, ref_lse = _both(q, k, v, qr, kr, ty, scale, cap, d)
        assert torch.equal(out, ref_out), name
        assert torch.equal(lse, ref_lse), name
