"""BlockMask-style block lists on the GPU: the list goes through
ffa_block_slices, then the forward and backward kernels; the oracle builds its
mask from the block list directly (cell by cell, and one slice per block for
the backward), never from the library's slices."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import O, check_grad, compare_out_lse, dev, ffa, say, to64

pytestmark = pytest.mark.gpu


def _local_global(n_qb, n_kb, window):
    num = np.zeros(n_qb, np.int32)
    idx = np.zeros((n_qb, window + 1), np.int32)
    for b in range(n_qb):
        blocks = sorted({0} | set(range(max(0, b - window + 1), min(b, n_kb - 1) + 1)))
        num[b] = len(blocks)
        idx[b, :len(blocks)] = blocks[::-1]
    return num, idx


def _random(rng, n_qb, n_kb, density):
    num = np.zeros(n_qb, np.int32)
    idx = np.zeros((n_qb, n_kb), np.int32)
    for b in range(n_qb):
        listed = rng.permutation(n_kb)[: int(rng.binomial(n_kb, density))]
        num[b] = listed.size
        idx[b, :listed.size] = listed
    return num, idx


CASES = [
    # (name, T, hq, hkv, d, block, softcap)
    ("local_global", 2048 - 37, 4, 2, 128, 128, 0.0),
    ("random", 1500, 2, 1, 64, 64, 10.0),
    ("random", 777, 4, 4, 128, 32, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_T{c[1]}_d{c[4]}_b{c[5]}" for c in CASES])
def test_block_list_fwd_bwd(case):
    name, T, hq, hkv, d, blk, cap = case
    say(f"block list {case}")
    rng = np.random.default_rng(T)
    nb = -(-T // blk)
    num, idx = _local_global(nb, nb, 3) if name == "local_global" else _random(rng, nb, nb, 0.3)
    qr, kr, ty = ffa.ffa_block_slices(num, idx, T, T, blk, blk)
    q, k, v, do = W.make_tensors(T, T, hq, hkv, d, seed=int(T) + 1)
    scale = d ** -0.5
    dv_ = dev()
    qd, kd, vd, od = q.to(dv_), k.to(dv_), v.to(dv_), do.to(dv_)
    out, lse = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, cap)
    dq, dk, dv = ffa.ffa_bwd(qd, kd, vd, out, lse, od, qr, kr, ty, scale, cap)
    torch.cuda.synchronize()
    vis = O.block_visibility(num, idx, blk, blk, T, T)
    ref_out, ref_lse = O.attention_fwd_masked(to64(q), to64(k), to64(v), vis, scale, cap)
    e_out, e_lse = compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, str(case))
    pqr, pkr, pty = O.block_slices_plain(num, idx, blk, blk, T, T)
    rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), pqr, pkr, pty, scale, cap,
                                       magnitudes=True)
    errs = [check_grad(n, g, r, str(case), m)
            for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags)]
    say(f"  {qr.shape[0]} slices; out {e_out:.3e} lse {e_lse:.3e} dq/dk/dv {errs[0]:.3e} {errs[1]:.3e} {errs[2]:.3e}")
