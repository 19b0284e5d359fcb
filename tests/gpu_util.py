"""Shared helpers for the GPU parity tests (inputs, oracle calls, comparisons).

Every comparison made through ``compare_out_lse`` and ``check_grad`` is also
written to a parity record (one entry per test and output: the max-abs error,
max |ref| and their ratio), saved as JSON when the session ends; see
``conftest.py``.
"""
import os
import sys

import numpy as np
import torch

import workloads as W  # noqa: F401  (re-exported for the tests)
from _lib import ensure_built, ffa
from oracle import ffa_oracle as O

OUT_TOL = 2e-2    # max-abs on bf16 out
LSE_TOL = 1e-3    # max-abs on fp32 lse
# dq, dk, dv: the out tolerance read plainly, 2e-2 max-abs per element, plus
# the rounding of the result to bf16 where that alone can come near it.  bf16
# keeps 8 significant bits, so rounding x to nearest moves it by up to half
# an ulp, 2^(floor(log2|x|) - 8) <= 2^-8 |x| (the unit roundoff); from
# |x| = 8 on that exceeds 2e-2 by itself, so no bf16 result could meet a bare
# 2e-2 there.  The half-ulp term is added where |ref| >= 4 and nowhere else.
GRAD_TOL_ABS = 2e-2
GRAD_HALF_ULP = 2.0 ** -8
GRAD_HALF_ULP_FROM = 4.0

# (test id, what, field) -> value; see record()
PARITY = []


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    ensure_built()
    return torch.device("cuda:0")


def to64(t):
    return t.double().numpy() if t is not None else None


def _np(x):
    if hasattr(x, "detach"):
        return x.detach().double().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def _test_id():
    return os.environ.get("PYTEST_CURRENT_TEST", "?").split(" (")[0]


def record(ctx, name, err, ref_max, tol, n, excess):
    """Add one comparison to the parity record: the max-abs error, max |ref|,
    their ratio, and the largest (error - bound) over the elements (<= 0
    passes)."""
    PARITY.append({
        "test": _test_id(), "ctx": str(ctx), "output": name, "max_abs": float(err),
        "max_ref": float(ref_max), "rel_to_max_ref": float(err / ref_max) if ref_max > 0 else 0.0,
        "tol": tol, "excess": float(excess), "n": int(n),
    })


def sample_rows(Tq, rng, n=96, extra=()):
    """Rows spread over the tensor, plus tile edges and the given extras."""
    base = set(int(x) for x in rng.integers(0, Tq, size=n))
    for r in (0, 1, 127, 128, Tq - 1, Tq - 2) + tuple(extra):
        if 0 <= r < Tq:
            base.add(int(r))
    return np.array(sorted(base))


def compare_out_lse(out, lse, ref_out, ref_lse, ctx=""):
    out = _np(out)
    lse = _np(lse)
    inf_gpu, inf_ref = np.isneginf(lse), np.isneginf(ref_lse)
    assert np.array_equal(inf_gpu, inf_ref), f"{ctx}: -inf lse rows differ"
    fin = ~inf_ref
    err_lse = float(np.abs(lse[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    err_out = float(np.abs(out - ref_out).max()) if out.size else 0.0
    record(ctx, "out", err_out, float(np.abs(ref_out).max()) if out.size else 0.0, OUT_TOL, out.size,
           err_out - OUT_TOL)
    record(ctx, "lse", err_lse, float(np.abs(ref_lse[fin]).max()) if fin.any() else 0.0, LSE_TOL, int(fin.sum()),
           err_lse - LSE_TOL)
    assert np.all(out[inf_ref] == 0.0), f"{ctx}: rows with no visible key must be 0"
    assert err_out <= OUT_TOL, f"{ctx}: out max-abs {err_out}"
    assert err_lse <= LSE_TOL, f"{ctx}: lse max-abs {err_lse}"
    return err_out, err_lse


def grad_tol(ref):
    """Per-element bound for a bf16 gradient: 2e-2, plus the bf16 half-ulp
    bound 2^-8 |ref| where |ref| >= 4."""
    a = np.abs(ref)
    return GRAD_TOL_ABS + np.where(a >= GRAD_HALF_ULP_FROM, GRAD_HALF_ULP * a, 0.0)


def check_grad(name, got, ref, ctx="", mag=None):
    """Element-wise |got - ref| <= grad_tol(ref); returns the max-abs error.

    ``mag`` (the oracle's sum of |terms| per element) is only reported: the
    ratio of the error to 2^-8 * mag says how much of a worst-case rounding
    budget a case used.
    """
    got = _np(got)
    ref = np.asarray(ref, dtype=np.float64)
    if not got.size:
        return 0.0
    diff = np.abs(got - ref)
    err = float(diff.max())
    ref_max = float(np.abs(ref).max())
    excess = float((diff - grad_tol(ref)).max())
    record(ctx, name, err, ref_max, "2e-2 + 2^-8 |ref| where |ref| >= 4", got.size, excess)
    if mag is not None:
        budget = float((diff / (2.0 ** -8 * np.asarray(mag) + 1e-30)).max())
        PARITY[-1]["err_over_term_budget"] = budget
    assert excess <= 0.0, f"{ctx}: {name} max-abs {err} (max |ref| {ref_max})"
    return err


def check_grads(got3, ref3, ctx="", mags=None):
    """check_grad over (dq, dk, dv); returns the three max-abs errors."""
    mags = mags if mags is not None else (None, None, None)
    return [check_grad(n, g, r, ctx, m) for n, g, r, m in zip(("dq", "dk", "dv"), got3, ref3, mags)]


def run_fwd(q, k, v, qr, kr, ty, scale, softcap, device):
    qd, kd, vd = q.to(device), k.to(device), v.to(device)
    out, lse = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, softcap)
    torch.cuda.synchronize()
    return out, lse
