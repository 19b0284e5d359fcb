"""PyTorch custom operators over the C ABI, so the path runs under torch.compile.

The MagiAttention issue on dummy/padded attention slices is about exactly this
use: ``flex_flash_attn_func`` inside ``torch.compile`` with static shapes,
obtained by padding the slice list with empty ``[x, x]`` slices up to a fixed
count.  The flash-attention pull request "Add torch.compile support to flash
attention 3" shows the mechanism: register the kernels as custom operators with
fake implementations (output shapes only) and an autograd formula.

Here ``ffa_amd::fwd`` returns ``(out, lse, saved)`` and ``ffa_amd::bwd`` returns
``(dq, dk, dv)``.  ``saved`` is the training forward's record for the backward
(out's bf16 rounding residual, for the row term D = rowsum(dO * out), and the
fp16 copy of v): a uint8 tensor, filled only when ``train`` is true (a backward
may follow), else empty, and then the backward re-runs the training forward
to get one.  The compiler treats both as opaque; their fake
implementations depend only on tensor shapes, so one compiled graph serves every
slice list of the same padded length.  The real implementations call the C ABI
through the ctypes binding (slice tensors on the GPU are copied to the host
there: one synchronisation).  ``lse`` is returned without a gradient, as in the
eager autograd path.  The optional ``alibi_slopes`` (fp32 [hq] on the GPU: a
distance bias ``slope[h] * (j - i)`` on the scores) takes no gradient either.

Plans come from the binding's plan cache (``cached_plan``), so a mask shared by
many layers and steps is planned on the host once; with the cache turned off
(``FFA_PLAN_CACHE=0``) every call plans for itself through the one-shot entry
points.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import cached_plan as _cached_plan
from . import ffa_bwd as _ffa_bwd
from . import ffa_bwd_planned as _ffa_bwd_planned
from . import ffa_fwd as _ffa_fwd
from . import ffa_fwd_planned as _ffa_fwd_planned

NAMESPACE = "ffa_amd"


def _saved_bytes(q, k):
    from . import ffa_saved_size
    return max(ffa_saved_size(q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2]), 16)


@torch.library.custom_op(f"{NAMESPACE}::fwd", mutates_args=(), device_types="cuda")
def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_ranges: torch.Tensor,
        k_ranges: torch.Tensor, attn_type_map: torch.Tensor, scale: float,
        softcap: float, alibi_slopes: Optional[torch.Tensor] = None,
        train: bool = False) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    plan = _cached_plan(q.shape[0], k.shape[0], q_ranges, k_ranges, attn_type_map, q.device)
    if plan is None:
        r = _ffa_fwd(q, k, v, q_ranges, k_ranges, attn_type_map, scale, softcap, alibi_slopes=alibi_slopes,
                     train=train)
    else:
        r = _ffa_fwd_planned(plan, q, k, v, scale, softcap, alibi_slopes=alibi_slopes, train=train)
    return (r[0], r[1], r[2] if train else q.new_empty((0,), dtype=torch.uint8))


@fwd.register_fake
def _fwd_fake(q, k, v, q_ranges, k_ranges, attn_type_map, scale, softcap, alibi_slopes=None, train=False):
    torch._check(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, lambda: "q, k, v must be [T, heads, d]")
    n = _saved_bytes(q, k) if train else 0
    return (torch.empty_like(q), q.new_empty((q.shape[0], q.shape[1]), dtype=torch.float32),
            q.new_empty((n,), dtype=torch.uint8))


@torch.library.custom_op(f"{NAMESPACE}::bwd", mutates_args=(), device_types="cuda")
def bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
        lse: torch.Tensor, saved: torch.Tensor, q_ranges: torch.Tensor, k_ranges: torch.Tensor,
        attn_type_map: torch.Tensor, scale: float, softcap: float,
        alibi_slopes: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    rec = saved if saved.numel() else None
    plan = _cached_plan(q.shape[0], k.shape[0], q_ranges, k_ranges, attn_type_map, q.device)
    if plan is None:
        return _ffa_bwd(q, k, v, out, lse, dout.contiguous(), q_ranges, k_ranges, attn_type_map,
                        scale, softcap, alibi_slopes=alibi_slopes, saved=rec)
    return _ffa_bwd_planned(plan, q, k, v, out, lse, dout.contiguous(), scale, softcap,
                            alibi_slopes=alibi_slopes, saved=rec)


@bwd.register_fake
def _bwd_fake(dout, q, k, v, out, lse, saved, q_ranges, k_ranges, attn_type_map, scale, softcap,
              alibi_slopes=None):
    return torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)


def _setup_context(ctx, inputs, output):
    q, k, v, q_ranges, k_ranges, attn_type_map, scale, softcap, alibi_slopes, train = inputs
    out, lse, saved = output
    ctx.save_for_backward(q, k, v, out, lse, saved, q_ranges, k_ranges, attn_type_map, alibi_slopes)
    ctx.scale, ctx.softcap = scale, softcap
    ctx.mark_non_differentiable(lse, saved)


def _backward(ctx, dout, dlse, dsaved):
    q, k, v, out, lse, saved, q_ranges, k_ranges, attn_type_map, alibi_slopes = ctx.saved_tensors
    dq, dk, dv = bwd(dout, q, k, v, out, lse, saved, q_ranges, k_ranges, attn_type_map, ctx.scale,
                     ctx.softcap, alibi_slopes)
    return dq, dk, dv, None, None, None, None, None, None, None


fwd.register_autograd(_backward, setup_context=_setup_context)
