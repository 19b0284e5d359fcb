"""Shared helpers for the GPU parity tests (inputs, oracle calls, comparisons)."""
import sys

import numpy as np
import torch

import workloads as W
from _lib import ensure_built, ffa
from oracle import ffa_oracle as O

OUT_TOL = 2e-2    # max-abs on bf16 out
LSE_TOL = 1e-3    # max-abs on fp32 lse
# dq, dk, dv: no tolerance is fixed for them.  From the arithmetic: each is a
# sum of terms whose factors P and dS enter the matrix cores rounded to bf16
# (relative error <= u = 2^-8 per term, so <= u * sum|terms| for the sum), the
# row term D = rowsum(dO * out) is formed from the bf16 out (error <= u * A_i,
# see the oracle's magnitudes), and the result is rounded to bf16 once more
# (<= u * |ref|); 2e-2 absolute, as for out, covers fp32 accumulation:
#   |got - ref| <= 2e-2 + u * (|ref| + magnitude)
GRAD_TOL_ABS = 2e-2
GRAD_TOL_REL = 2.0 ** -8


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    ensure_built()
    return torch.device("cuda:0")


def to64(t):
    return t.double().numpy() if t is not None else None


def sample_rows(Tq, rng, n=96, extra=()):
    """Rows spread over the tensor, plus tile edges and the given extras."""
    base = set(int(x) for x in rng.integers(0, Tq, size=n))
    for r in (0, 1, 127, 128, Tq - 1, Tq - 2) + tuple(extra):
        if 0 <= r < Tq:
            base.add(int(r))
    return np.array(sorted(base))


def compare_out_lse(out, lse, ref_out, ref_lse, ctx=""):
    out = out.double().cpu().numpy() if hasattr(out, "cpu") else out
    lse = lse.double().cpu().numpy() if hasattr(lse, "cpu") else lse
    inf_gpu, inf_ref = np.isneginf(lse), np.isneginf(ref_lse)
    assert np.array_equal(inf_gpu, inf_ref), f"{ctx}: -inf lse rows differ"
    fin = ~inf_ref
    err_lse = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    err_out = float(np.abs(out - ref_out).max()) if out.size else 0.0
    assert np.all(out[inf_ref] == 0.0), f"{ctx}: rows with no visible key must be 0"
    assert err_out <= OUT_TOL, f"{ctx}: out max-abs {err_out}"
    assert err_lse <= LSE_TOL, f"{ctx}: lse max-abs {err_lse}"
    return err_out, err_lse


def run_fwd(q, k, v, qr, kr, ty, scale, softcap, device):
    qd, kd, vd = q.to(device), k.to(device), v.to(device)
    out, lse = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, softcap)
    torch.cuda.synchronize()
    return out, lse
