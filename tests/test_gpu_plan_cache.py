"""The binding's plan cache: flex_flash_attn_func (and the custom operators)
plan a slice list once per (device, stream, sizes, slices) and reuse it; the
results equal the one-shot entry points bitwise."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, ffa, say

pytestmark = pytest.mark.gpu


def _lists(w):
    qr, kr, ty = w.slices()
    # the same mask with other padding, and a different mask
    qr2 = np.concatenate([qr, [[5, 5]]]).astype(np.int32)
    kr2 = np.concatenate([kr, [[0, 0]]]).astype(np.int32)
    ty2 = np.concatenate([ty, [0]]).astype(np.int32)
    qr3, kr3, ty3 = np.array([[0, w.Tq]], np.int32), np.array([[0, w.Tk]], np.int32), np.array([1], np.int32)
    return [(qr, kr, ty), (qr2, kr2, ty2), (qr3, kr3, ty3)]


def test_cache_hits_evicts_and_matches_one_shot():
    w = W.config(2)
    say("plan cache")
    q, k, v, do = W.workload_tensors(w)
    d = dev()
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    cache = ffa._PLAN_CACHE
    ffa.clear_plan_cache()
    old_capacity = cache.capacity
    cache.capacity = 2
    try:
        h0, m0 = cache.hits, cache.misses
        results = []
        for rep in range(2):
            for qr, kr, ty in _lists(w):
                qa, ka, va = (t.clone().requires_grad_() for t in (qd, kd, vd))
                out, lse = ffa.flex_flash_attn_func(qa, ka, va, qr, kr, ty, softmax_scale=w.scale)
                out.backward(od)
                results.append((out.detach(), lse, qa.grad, ka.grad, va.grad))
        torch.cuda.synchronize()
        # three lists through a two-plan cache, twice: every forward misses
        # (each list was evicted before it came back), every backward hits
        assert cache.misses - m0 == 6 and cache.hits - h0 == 6, (cache.misses - m0, cache.hits - h0)
        assert len(cache._plans) == 2
        for i, (qr, kr, ty) in enumerate(_lists(w)):
            o, l, rec = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, train=True)
            g = ffa.ffa_bwd(qd, kd, vd, o, l, od, qr, kr, ty, w.scale, saved=rec)
            torch.cuda.synchronize()
            for r in (results[i], results[i + 3]):
                assert torch.equal(r[0], o) and torch.equal(r[1], l)
                for a, b in zip(r[2:], g):
                    assert torch.equal(a, b)
        # another stream gets its own plan
        s = torch.cuda.Stream(device=d)
        with torch.cuda.stream(s):
            qr, kr, ty = _lists(w)[2]
            ffa.flex_flash_attn_func(qd, kd, vd, qr, kr, ty, softmax_scale=w.scale)
        s.synchronize()
        assert cache.misses - m0 == 7
    finally:
        torch.cuda.synchronize()
        ffa.clear_plan_cache()
        cache.capacity = old_capacity
