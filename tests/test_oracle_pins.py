"""Pins for the CPU oracle: each test ties it to something other than itself.

Library routines (torch SDPA in float64, its lower-right causal bias, scipy's
logsumexp, torch autograd), closed forms, brute force over cells and the
printed result of the pages' repro script.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import workloads as W
from oracle import ffa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng_seed = 1234


def _rand(shape, rng):
    # bf16-representable values, like the real inputs
    x = torch.from_numpy(rng.standard_normal(shape)).to(torch.bfloat16)
    return x.double().numpy()


def _sdpa(q, k, v, scale, mask=None, is_causal=False):
    """torch SDPA in float64 on [T, h, d] arrays (one batch)."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=is_causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


# ---------------------------------------------------------------- mask semantics
def _brute_visible(i, j, q_ranges, k_ranges, types):
    n = 0
    for (qs, qe), (ks, ke), t in zip(q_ranges, k_ranges, types):
        if qs == qe or ks == ke:
            continue
        if not (qs <= i < qe and ks <= j < ke):
            continue
        # CAUSAL: the diagonal passes through the slice's bottom-right corner:
        # the last query row sees the last key, and a key must lie at least as
        # far from the k end as the row lies from the q end
        if t == O.CAUSAL and (ke - 1 - j) < (qe - 1 - i):
            continue
        n += 1
    return n


def test_mask_brute_force_tiny():
    rng = np.random.default_rng(0)
    for trial in range(40):
        Tq, Tk = int(rng.integers(1, 24)), int(rng.integers(1, 24))
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=4, n_dummies=2)
        sl = O.normalise_slices(qr, kr, ty, Tq, Tk)
        M = O.visibility(sl, np.arange(Tq), np.arange(Tk))
        for i in range(Tq):
            for j in range(Tk):
                assert M[i, j] == _brute_visible(i, j, qr.tolist(), kr.tolist(), ty.tolist())


def test_pages_example_is_prefix_lm():
    """The repro's two slices give: first half bidirectional, second half causal."""
    g = json.load(open(os.path.join(GOLDEN, "pages_repro.json")))
    T, half = g["total_seqlen"], g["total_seqlen"] // 2
    sl = O.normalise_slices(g["q_ranges"], g["k_ranges"], g["attn_type_map"], T, T)
    M = O.visibility(sl, np.arange(T), np.arange(T))
    i, j = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    expect = np.where(i < half, j < half, j <= i)
    assert np.array_equal(M > 0, expect)
    assert M.max() == 1


def test_bottom_right_causal_matches_lower_right_bias():
    from torch.nn.attention.bias import causal_lower_right
    rng = np.random.default_rng(3)
    for Lq, Lk in [(5, 9), (17, 40), (33, 33)]:
        q, k, v = _rand((Lq, 2, 8), rng), _rand((Lk, 2, 8), rng), _rand((Lk, 2, 8), rng)
        out, _ = O.attention_fwd(q, k, v, [[0, Lq]], [[0, Lk]], [O.CAUSAL], 0.3)
        bias = causal_lower_right(Lq, Lk)
        ref = _sdpa(q, k, v, 0.3, mask=bias._materialize(torch.device("cpu")))
        np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_short_k_causal_leaves_top_rows_empty():
    """CAUSAL slice with fewer keys than queries: the top rows see nothing."""
    rng = np.random.default_rng(4)
    Lq, Lk = 12, 5
    q, k, v = _rand((Lq, 1, 4), rng), _rand((Lk, 1, 4), rng), _rand((Lk, 1, 4), rng)
    out, lse = O.attention_fwd(q, k, v, [[0, Lq]], [[0, Lk]], [O.CAUSAL], 0.5)
    # row i sees keys j <= i - (Lq - Lk): rows 0..6 see none
    assert np.all(out[:Lq - Lk] == 0.0) and np.all(lse[:Lq - Lk] == -np.inf)
    assert np.all(np.isfinite(lse[Lq - Lk:]))


# ---------------------------------------------------------------- forward values
def test_brute_force_forward_tiny():
    rng = np.random.default_rng(5)
    for trial in range(12):
        Tq, Tk, d = int(rng.integers(1, 10)), int(rng.integers(1, 10)), 3
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=3, n_dummies=1)
        q, k, v = _rand((Tq, 2, d), rng), _rand((Tk, 1, d), rng), _rand((Tk, 1, d), rng)
        cap = [0.0, 1.5][trial % 2]
        out, lse = O.attention_fwd(q, k, v, qr, kr, ty, 0.7, softcap=cap)
        for h in range(2):
            for i in range(Tq):
                scores = []
                for j in range(Tk):
                    if _brute_visible(i, j, qr.tolist(), kr.tolist(), ty.tolist()):
                        x = 0.7 * sum(q[i, h, c] * k[j, 0, c] for c in range(d))
                        if cap:
                            x = cap * math.tanh(x / cap)
                        scores.append((x, j))
                if not scores:
                    assert lse[i, h] == -math.inf and np.all(out[i, h] == 0)
                    continue
                mx = max(x for x, _ in scores)
                den = sum(math.exp(x - mx) for x, _ in scores)
                num = [sum(math.exp(x - mx) * v[j, 0, c] for x, j in scores) for c in range(d)]
                assert abs(lse[i, h] - (mx + math.log(den))) < 1e-12
                np.testing.assert_allclose(out[i, h], np.array(num) / den, rtol=1e-12, atol=1e-13)


def test_single_causal_slice_is_textbook_causal():
    rng = np.random.default_rng(6)
    T = 300
    q, k, v = _rand((T, 3, 16), rng), _rand((T, 3, 16), rng), _rand((T, 3, 16), rng)
    out, _ = O.attention_fwd(q, k, v, [[0, T]], [[0, T]], [O.CAUSAL], 0.25)
    ref = _sdpa(q, k, v, 0.25, is_causal=True)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_single_full_slice_is_dense_softmax():
    rng = np.random.default_rng(7)
    Tq, Tk = 70, 130
    q, k, v = _rand((Tq, 2, 32), rng), _rand((Tk, 2, 32), rng), _rand((Tk, 2, 32), rng)
    out, _ = O.attention_fwd(q, k, v, [[0, Tq]], [[0, Tk]], [O.FULL], 1 / math.sqrt(32))
    ref = _sdpa(q, k, v, 1 / math.sqrt(32))
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_gqa_is_repeat_interleave():
    rng = np.random.default_rng(8)
    T, hq, hkv = 96, 8, 2
    q, k, v = _rand((T, hq, 8), rng), _rand((T, hkv, 8), rng), _rand((T, hkv, 8), rng)
    out, _ = O.attention_fwd(q, k, v, [[0, T]], [[0, T]], [O.CAUSAL], 0.4)
    kr = np.repeat(k, hq // hkv, axis=1)
    vr = np.repeat(v, hq // hkv, axis=1)
    ref = _sdpa(q, kr, vr, 0.4, is_causal=True)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_packed_docs_equal_per_doc_attention():
    rng = np.random.default_rng(9)
    lens = [37, 64, 5, 120, 1]
    T = sum(lens)
    q, k, v = _rand((T, 2, 16), rng), _rand((T, 2, 16), rng), _rand((T, 2, 16), rng)
    spans, s = [], 0
    for n in lens:
        spans.append([s, s + n]); s += n
    out, _ = O.attention_fwd(q, k, v, spans, spans, [O.CAUSAL] * len(spans), 0.3)
    for a, b in spans:
        ref = _sdpa(q[a:b], k[a:b], v[a:b], 0.3, is_causal=True)
        np.testing.assert_allclose(out[a:b], ref, rtol=1e-11, atol=1e-12)


def test_lse_is_logsumexp_of_visible_scores():
    rng = np.random.default_rng(10)
    Tq, Tk = 50, 80
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=5)
    q, k, v = _rand((Tq, 1, 8), rng), _rand((Tk, 1, 8), rng), _rand((Tk, 1, 8), rng)
    _, lse = O.attention_fwd(q, k, v, qr, kr, ty, 0.6)
    vis = O.visibility(O.normalise_slices(qr, kr, ty, Tq, Tk), np.arange(Tq), np.arange(Tk)) > 0
    scores = 0.6 * (torch.from_numpy(q[:, 0]) @ torch.from_numpy(k[:, 0]).T).numpy()
    for i in range(Tq):
        if not vis[i].any():
            assert lse[i, 0] == -np.inf
        else:
            assert abs(lse[i, 0] - logsumexp(scores[i, vis[i]])) < 1e-12


def test_dummies_change_nothing_bitwise():
    """The pages' repro: padding with [0,0] type-0 rows gives a 0.0 max rel diff."""
    g = json.load(open(os.path.join(GOLDEN, "pages_repro.json")))
    rng = np.random.default_rng(11)
    T = 256  # the repro's slice pattern at a tenth of the size
    qr = np.array(g["q_ranges"]) * T // g["total_seqlen"]
    kr = np.array(g["k_ranges"]) * T // g["total_seqlen"]
    ty = np.array(g["attn_type_map"])
    q, k, v = _rand((T, 4, 8), rng), _rand((T, 1, 8), rng), _rand((T, 1, 8), rng)
    base, base_lse = O.attention_fwd(q, k, v, qr, kr, ty, 0.35)
    pq, pk, pt = W.pad_slices(qr, kr, ty, g["max_num_slices"])
    padded, padded_lse = O.attention_fwd(q, k, v, pq, pk, pt, 0.35)
    num = np.abs(base - padded)
    den = np.maximum(np.maximum(np.abs(base), np.abs(padded)), g["max_rel_diff_eps"])
    assert float((num / den).max()) == g["printed"]["out_max_rel_diff"]
    assert np.array_equal(base_lse, padded_lse)
    # dummies of either kind, anywhere in the list, either type
    for seed in range(5):
        r2 = np.random.default_rng(seed)
        qx, kx, tx = list(map(list, qr)), list(map(list, kr)), list(ty)
        for _ in range(4):
            pos = int(r2.integers(0, len(qx) + 1))
            x = int(r2.integers(0, T + 1))
            dq_, dk_ = ([x, x], [0, T]) if r2.random() < 0.5 else ([0, T], [x, x])
            qx.insert(pos, dq_); kx.insert(pos, dk_); tx.insert(pos, int(r2.integers(0, 2)))
        o2, l2 = O.attention_fwd(q, k, v, qx, kx, tx, 0.35)
        assert np.array_equal(o2, base) and np.array_equal(l2, base_lse)


def test_rows_with_no_visible_key():
    rng = np.random.default_rng(12)
    T = 40
    q, k, v = _rand((T, 2, 4), rng), _rand((T, 1, 4), rng), _rand((T, 1, 4), rng)
    out, lse = O.attention_fwd(q, k, v, [[0, 10], [25, 40]], [[0, 10], [5, 30]], [1, 0], 0.5)
    assert np.all(out[10:25] == 0.0) and np.all(lse[10:25] == -np.inf)
    out, lse = O.attention_fwd(q, k, v, np.zeros((3, 2)), np.zeros((3, 2)), [0, 1, 0], 0.5)
    assert np.all(out == 0.0) and np.all(lse == -np.inf)


def test_softcap_limits():
    rng = np.random.default_rng(13)
    T = 64
    q, k, v = _rand((T, 2, 16), rng), _rand((T, 2, 16), rng), _rand((T, 2, 16), rng)
    qr, kr, ty = [[0, 32], [32, 64]], [[0, 32], [0, 64]], [0, 1]
    # a huge cap is the identity on the logits
    a, la = O.attention_fwd(q, k, v, qr, kr, ty, 0.25, softcap=1e6)
    b, lb = O.attention_fwd(q, k, v, qr, kr, ty, 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(la, lb, rtol=1e-9, atol=1e-10)
    # a tiny cap squashes every logit to ~0: plain average of the visible values
    c, lc = O.attention_fwd(q, k, v, qr, kr, ty, 0.25, softcap=1e-7)
    vis = O.visibility(O.normalise_slices(qr, kr, ty, T, T), np.arange(T), np.arange(T)) > 0
    for i in range(T):
        np.testing.assert_allclose(c[i], v[vis[i]].mean(axis=0), rtol=1e-6, atol=1e-6)
        assert abs(lc[i, 0] - math.log(vis[i].sum())) < 1e-6
    # saturation: scores far beyond the cap land on +-cap
    cap = 2.0
    q1 = np.array([[[1.0]]])
    k1 = np.array([[[1e4]], [[-1e4]]])
    v1 = np.array([[[3.0]], [[-5.0]]])
    o1, l1 = O.attention_fwd(q1, k1, v1, [[0, 1]], [[0, 2]], [0], 1.0, softcap=cap)
    w = math.exp(cap) / (math.exp(cap) + math.exp(-cap))
    assert abs(o1[0, 0, 0] - (3.0 * w - 5.0 * (1 - w))) < 1e-12
    assert abs(l1[0, 0] - math.log(math.exp(cap) + math.exp(-cap))) < 1e-12


def test_sampled_rows_match_full():
    rng = np.random.default_rng(14)
    T = 200
    qr, kr, ty = W.random_slices(rng, T, T, max_slices=6, n_dummies=2)
    q, k, v = _rand((T, 4, 8), rng), _rand((T, 2, 8), rng), _rand((T, 2, 8), rng)
    full, lfull = O.attention_fwd(q, k, v, qr, kr, ty, 0.3, softcap=5.0)
    rows = np.array([0, 7, 63, 64, 150, 199])
    part, lpart = O.attention_fwd(q, k, v, qr, kr, ty, 0.3, softcap=5.0, rows=rows)
    assert np.array_equal(part, full[rows]) and np.array_equal(lpart, lfull[rows])


def test_invalid_slices_raise():
    for qr, kr, ty in [([[5, 3]], [[0, 4]], [0]), ([[0, 4]], [[0, 99]], [0]),
                       ([[0, 4]], [[0, 4]], [2]), ([[-1, 4]], [[0, 4]], [1])]:
        with pytest.raises(ValueError):
            O.normalise_slices(qr, kr, ty, 10, 10)


# ---------------------------------------------------------------- backward
def _f(q, k, v, do, qr, kr, ty, scale, cap):
    out, _ = O.attention_fwd(q, k, v, qr, kr, ty, scale, softcap=cap)
    return float((out * do).sum())


@pytest.mark.parametrize("cap", [0.0, 0.8])
def test_backward_finite_differences(cap):
    rng = np.random.default_rng(15)
    Tq, Tk, d = 20, 18, 4
    qr, kr, ty = [[0, 8], [8, 20], [8, 20], [3, 3]], [[0, 10], [0, 4], [6, 18], [0, 18]], [1, 0, 1, 0]
    q, k, v = _rand((Tq, 2, d), rng), _rand((Tk, 1, d), rng), _rand((Tk, 1, d), rng)
    do = _rand((Tq, 2, d), rng)
    dq, dk, dv = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.9, softcap=cap)
    eps = 1e-6
    for name, x, g in [("q", q, dq), ("k", k, dk), ("v", v, dv)]:
        for trial in range(3):
            delta = rng.standard_normal(x.shape)
            xp, xm = x + eps * delta, x - eps * delta
            args_p = dict(q=q, k=k, v=v); args_p[name] = xp
            args_m = dict(q=q, k=k, v=v); args_m[name] = xm
            fd = (_f(args_p["q"], args_p["k"], args_p["v"], do, qr, kr, ty, 0.9, cap)
                  - _f(args_m["q"], args_m["k"], args_m["v"], do, qr, kr, ty, 0.9, cap)) / (2 * eps)
            an = float((g * delta).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


@pytest.mark.parametrize("cap", [0.0, 3.0])
def test_backward_matches_autograd(cap):
    rng = np.random.default_rng(16)
    Tq, Tk, hq, hkv, d = 48, 56, 4, 2, 8
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=5, n_dummies=2)
    q, k, v = _rand((Tq, hq, d), rng), _rand((Tk, hkv, d), rng), _rand((Tk, hkv, d), rng)
    do = _rand((Tq, hq, d), rng)
    dq, dk, dv = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.5, softcap=cap)
    vis = torch.from_numpy(O.visibility(O.normalise_slices(qr, kr, ty, Tq, Tk),
                                        np.arange(Tq), np.arange(Tk)) > 0)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    kk = tk.repeat_interleave(hq // hkv, dim=1)
    vv = tv.repeat_interleave(hq // hkv, dim=1)
    u = 0.5 * torch.einsum("ihc,jhc->hij", tq, kk)
    s = cap * torch.tanh(u / cap) if cap else u
    s = s.masked_fill(~vis[None], float("-inf"))
    has = vis.any(dim=1)
    p = torch.softmax(torch.where(has[None, :, None], s, torch.zeros_like(s)), dim=-1)
    p = torch.where(vis[None], p, torch.zeros_like(p))
    out = torch.einsum("hij,jhc->ihc", p, vv)
    (out * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_backward_sampled_matches_full():
    rng = np.random.default_rng(17)
    T = 150
    qr, kr, ty = W.random_slices(rng, T, T, max_slices=5)
    q, k, v = _rand((T, 2, 8), rng), _rand((T, 1, 8), rng), _rand((T, 1, 8), rng)
    do = _rand((T, 2, 8), rng)
    dq, dk, dv = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.4, softcap=2.0)
    rows, keys = np.array([1, 50, 149]), np.array([0, 77, 140])
    sq, sk, sv = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.4, softcap=2.0, rows=rows, keys=keys)
    np.testing.assert_allclose(sq, dq[rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sk, dk[keys], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sv, dv[keys], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("cap", [0.0, 2.0])
def test_kv_head_subset_matches_autograd_on_those_heads(cap):
    """kv_heads=[g] computes only kv head g and the q heads reading it: the
    same numbers torch autograd gives on a problem that has only those heads
    (dk, dv of g sum over exactly those q heads), and the same as the rows of
    the all-heads result."""
    rng = np.random.default_rng(19)
    Tq, Tk, hq, hkv, d = 40, 52, 6, 3, 8
    grp = hq // hkv
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=5, n_dummies=1)
    q, k, v = _rand((Tq, hq, d), rng), _rand((Tk, hkv, d), rng), _rand((Tk, hkv, d), rng)
    do = _rand((Tq, hq, d), rng)
    g = 1
    hs = list(range(g * grp, (g + 1) * grp))
    out_s, lse_s = O.attention_fwd(q, k, v, qr, kr, ty, 0.45, cap, kv_heads=[g])
    dq_s, dk_s, dv_s = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.45, cap, kv_heads=[g])
    assert out_s.shape == (Tq, grp, d) and dk_s.shape == (Tk, 1, d)
    # against autograd on the sub-problem (q heads hs, kv head g alone)
    vis = torch.from_numpy(O.visibility(O.normalise_slices(qr, kr, ty, Tq, Tk),
                                        np.arange(Tq), np.arange(Tk)) > 0)
    tq = torch.from_numpy(q[:, hs]).requires_grad_()
    tk = torch.from_numpy(k[:, [g]]).requires_grad_()
    tv = torch.from_numpy(v[:, [g]]).requires_grad_()
    u = 0.45 * torch.einsum("ihc,jc->hij", tq, tk[:, 0])
    sc = cap * torch.tanh(u / cap) if cap else u
    sc = sc.masked_fill(~vis[None], float("-inf"))
    has = vis.any(dim=1)
    p = torch.softmax(torch.where(has[None, :, None], sc, torch.zeros_like(sc)), dim=-1)
    p = torch.where(vis[None], p, torch.zeros_like(p))
    out = torch.einsum("hij,jc->ihc", p, tv[:, 0])
    np.testing.assert_allclose(out_s, out.detach().numpy(), rtol=1e-11, atol=1e-12)
    (out * torch.from_numpy(do[:, hs])).sum().backward()
    np.testing.assert_allclose(dq_s, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk_s, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv_s, tv.grad.numpy(), rtol=1e-10, atol=1e-11)
    # and the all-heads result restricted to those heads, bitwise
    out_a, lse_a = O.attention_fwd(q, k, v, qr, kr, ty, 0.45, cap)
    dq_a, dk_a, dv_a = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.45, cap)
    assert np.array_equal(out_s, out_a[:, hs]) and np.array_equal(lse_s, lse_a[:, hs])
    assert np.array_equal(dq_s, dq_a[:, hs])
    assert np.array_equal(dk_s, dk_a[:, [g]]) and np.array_equal(dv_s, dv_a[:, [g]])


def test_visibility_skips_only_slices_that_add_nothing():
    """The visibility matrix of a row/column window equals the window cut out
    of the whole matrix, cell by cell against the brute-force rule."""
    rng = np.random.default_rng(20)
    T = 60
    qr, kr, ty = W.random_slices(rng, T, T, max_slices=6, n_dummies=2)
    sl = O.normalise_slices(qr, kr, ty, T, T)
    full = O.visibility(sl, np.arange(T), np.arange(T))
    for r0, r1, c0, c1 in ((0, 10, 0, 60), (17, 33, 5, 41), (50, 60, 50, 60), (30, 31, 0, 1)):
        rows, cols = np.arange(r0, r1), np.arange(c0, c1)
        win = O.visibility(sl, rows, cols)
        assert np.array_equal(win, full[r0:r1, c0:c1])
        for i in range(r0, r1):
            for j in range(c0, c1):
                assert bool(win[i - r0, j - c0]) == _brute_visible(i, j, qr, kr, ty)


# ---------------------------------------------------------------- tile lists
def _brute_tiles(qr, kr, ty, Tq, Tk, BM, BN):
    out = set()
    for r, ((qs, qe), (ks, ke), t) in enumerate(zip(qr, kr, ty)):
        for qt in range((Tq + BM - 1) // BM):
            for kt in range((Tk + BN - 1) // BN):
                c = 0
                for i in range(qt * BM, qt * BM + BM):
                    for j in range(kt * BN, kt * BN + BN):
                        if _brute_visible(i, j, [(qs, qe)], [(ks, ke)], [t]):
                            c += 1
                if c:
                    out.add((qt, kt, r, 0 if c == BM * BN else 1))
    return out


def test_tile_set_brute_force_small():
    rng = np.random.default_rng(18)
    for trial in range(10):
        Tq, Tk = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=4, n_dummies=1)
        BM, BN = [(8, 4), (4, 8), (16, 16)][trial % 3]
        assert O.tile_set(qr, kr, ty, Tq, Tk, BM, BN) == \
            _brute_tiles(qr.tolist(), kr.tolist(), ty.tolist(), Tq, Tk, BM, BN)


def test_tile_set_hand_example():
    # one CAUSAL slice over 256 tokens, 128 x 64 tiles:
    # q-tile 0 touches k-tiles 0, 1 on the diagonal (both partial);
    # q-tile 1 has k-tiles 0, 1 fully below the diagonal and 2, 3 on it.
    got = O.tile_set([[0, 256]], [[0, 256]], [1], 256, 256, 128, 64)
    assert got == {(0, 0, 0, 1), (0, 1, 0, 1), (1, 0, 0, 0), (1, 1, 0, 0), (1, 2, 0, 1), (1, 3, 0, 1)}
    # a k range ending inside a tile past the tensor end: that tile is partial
    got = O.tile_set([[0, 128]], [[0, 100]], [0], 128, 100, 128, 64)
    assert got == {(0, 0, 0, 0), (0, 1, 0, 1)}


def _kinds(ts):
    full = sum(1 for t in ts if t[3] == 0)
    return full, len(ts) - full


def test_tile_counts_closed_form():
    # tiny: FULL 128x128 slice -> 2 full tiles; causal second half -> 2 full + 2 partial
    w = W.config(1)
    assert _kinds(O.tile_set(*w.slices(), w.Tq, w.Tk, 128, 64)) == (4, 2)
    # long packed: per 8192-token causal document, q-tile t has 2t full + 2 diagonal tiles
    w = W.config(4)
    per_doc_full = sum(2 * t for t in range(64))
    assert _kinds(O.tile_set(*w.slices(), w.Tq, w.Tk, 128, 64)) == (8 * per_doc_full, 8 * 128)


@pytest.mark.parametrize("n,expect", [
    (1, 128 * 128 + sum(range(129, 257))),
    (2, 1024 * 1024 + sum(range(1025, 2049))),
    (4, 8 * 8192 * 8193 // 2),
    (5, 524800 + 31 * 524288 + (1049088 + 2097664 + 3146240 + 28 * 3670528)),
])
def test_visible_pairs_closed_form(n, expect):
    w = W.config(n)
    sl = O.normalise_slices(*w.slices(), w.Tq, w.Tk)
    if n in (4, 5):
        # count per slice rectangle (slices are disjoint), materialising each
        tot = 0
        for s in sl:
            _, qs, qe, ks, ke, t = s
            for r0 in range(qs, qe, 2048):
                rows = np.arange(r0, min(qe, r0 + 2048))
                tot += int(O.slice_cells(s, rows, np.arange(ks, ke)).sum())
        assert tot == expect
    else:
        assert O.visible_count(sl, w.Tq, w.Tk) == expect


def test_doc_config_closed_form():
    w = W.config(3)
    lens = W.doc_lengths()
    assert lens == [3523, 2702, 2219, 1292, 1438, 413, 544, 319, 929, 3005]
    sl = O.normalise_slices(*w.slices(), w.Tq, w.Tk)
    assert len(sl) == 10 and w.slices()[0].shape == (64, 2)
    assert O.visible_count(sl, w.Tq, w.Tk) == sum(n * (n + 1) // 2 for n in lens)


def test_backward_term_magnitudes_bound_the_gradients():
    """Triangle inequality, and equality when every term has one sign."""
    rng = np.random.default_rng(19)
    T = 90
    qr, kr, ty = W.random_slices(rng, T, T, max_slices=4)
    q, k, v = _rand((T, 2, 8), rng), _rand((T, 1, 8), rng), _rand((T, 1, 8), rng)
    do = _rand((T, 2, 8), rng)
    dq, dk, dv, (mq, mk, mv) = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.4, magnitudes=True)
    for g, m in ((dq, mq), (dk, mk), (dv, mv)):
        assert np.all(np.abs(g) <= m + 1e-12)
    # dO >= 0 and P >= 0: dv is a sum of non-negative terms, so it equals its magnitude
    _, _, dv2, (_, _, mv2) = O.attention_bwd(q, k, v, np.abs(do), qr, kr, ty, 0.4, magnitudes=True)
    np.testing.assert_allclose(dv2, mv2, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- distance bias (ALiBi)
def test_alibi_closed_form_zero_queries():
    """q = 0: every score is the bias m (j - i), so over keys [0, n) the weights
    are e^{m j} / sum_j e^{m j} for every row, and
    lse_i = -m i + log((e^{m n} - 1) / (e^m - 1))."""
    rng = np.random.default_rng(40)
    Tq, n, d = 9, 13, 4
    slopes = np.array([0.25, -0.125, 0.5])
    q = np.zeros((Tq, 3, d))
    k, v = _rand((n, 1, d), rng), _rand((n, 1, d), rng)
    out, lse = O.attention_fwd(q, k, v, [[0, Tq]], [[0, n]], [O.FULL], 0.7, alibi_slopes=slopes)
    for h, m in enumerate(slopes):
        w = np.array([math.exp(m * j) for j in range(n)])
        w /= w.sum()
        for i in range(Tq):
            assert abs(lse[i, h] - (-m * i + math.log(math.expm1(m * n) / math.expm1(m)))) < 1e-12
            np.testing.assert_allclose(out[i, h], w @ v[:, 0], rtol=0, atol=1e-13)


def test_alibi_causal_matches_sdpa_float_mask():
    """One causal slice over the whole sequence with ALiBi slopes 2^(-8h/H):
    torch SDPA with the bias (and -inf above the diagonal) as a float mask."""
    rng = np.random.default_rng(41)
    T, hq, hkv, d = 70, 4, 2, 16
    slopes = np.array([2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)])
    q, k, v = _rand((T, hq, d), rng), _rand((T, hkv, d), rng), _rand((T, hkv, d), rng)
    out, lse = O.attention_fwd(q, k, v, [[0, T]], [[0, T]], [O.CAUSAL], 0.3, alibi_slopes=slopes)
    i = torch.arange(T, dtype=torch.float64)[:, None]
    j = torch.arange(T, dtype=torch.float64)[None, :]
    above = j > i
    mask = torch.stack([torch.where(above, float("-inf"), float(m) * (j - i)) for m in slopes])[None]
    kr = np.repeat(k, hq // hkv, axis=1)
    vr = np.repeat(v, hq // hkv, axis=1)
    np.testing.assert_allclose(out, _sdpa(q, kr, vr, 0.3, mask=mask), rtol=1e-10, atol=1e-12)
    scores = 0.3 * np.einsum("ihc,jhc->hij", q, kr) + mask[0].numpy()
    np.testing.assert_allclose(lse, logsumexp(scores, axis=-1).T, rtol=1e-12, atol=1e-12)


def test_alibi_zero_slopes_change_nothing():
    rng = np.random.default_rng(42)
    T, d = 60, 8
    qr, kr, ty = W.random_slices(rng, T, T, max_slices=5)
    q, k, v = _rand((T, 2, d), rng), _rand((T, 1, d), rng), _rand((T, 1, d), rng)
    a = O.attention_fwd(q, k, v, qr, kr, ty, 0.4, softcap=2.0)
    b = O.attention_fwd(q, k, v, qr, kr, ty, 0.4, softcap=2.0, alibi_slopes=[0.0, 0.0])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("cap", [0.0, 3.0])
def test_alibi_backward_matches_autograd(cap):
    """Bias added after the softcap: dense masked formula under torch autograd."""
    rng = np.random.default_rng(43)
    Tq, Tk, hq, hkv, d = 40, 52, 4, 2, 8
    slopes = np.array([0.3, -0.2, 0.05, 0.0])
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=5, n_dummies=1)
    q, k, v = _rand((Tq, hq, d), rng), _rand((Tk, hkv, d), rng), _rand((Tk, hkv, d), rng)
    do = _rand((Tq, hq, d), rng)
    dq, dk, dv = O.attention_bwd(q, k, v, do, qr, kr, ty, 0.5, softcap=cap, alibi_slopes=slopes)
    vis = torch.from_numpy(O.visibility(O.normalise_slices(qr, kr, ty, Tq, Tk),
                                        np.arange(Tq), np.arange(Tk)) > 0)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    kk = tk.repeat_interleave(hq // hkv, dim=1)
    vv = tv.repeat_interleave(hq // hkv, dim=1)
    u = 0.5 * torch.einsum("ihc,jhc->hij", tq, kk)
    s = cap * torch.tanh(u / cap) if cap else u
    dist = (torch.arange(Tk, dtype=torch.float64)[None, :] - torch.arange(Tq, dtype=torch.float64)[:, None])
    s = s + torch.from_numpy(slopes)[:, None, None] * dist[None]
    s = s.masked_fill(~vis[None], float("-inf"))
    has = vis.any(dim=1)
    p = torch.softmax(torch.where(has[None, :, None], s, torch.zeros_like(s)), dim=-1)
    p = torch.where(vis[None], p, torch.zeros_like(p))
    out = torch.einsum("hij,jhc->ihc", p, vv)
    (out * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-11)
    o_ref, _ = O.attention_fwd(q, k, v, qr, kr, ty, 0.5, softcap=cap, alibi_slopes=slopes)
    np.testing.assert_allclose(o_ref, out.detach().numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- block lists
def test_block_visibility_brute_force():
    rng = np.random.default_rng(50)
    for trial in range(20):
        Tq, Tk = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        bq, bk = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        nqb, nkb = -(-Tq // bq), -(-Tk // bk)
        width = int(rng.integers(1, nkb + 1))
        num = rng.integers(0, width + 1, nqb)
        idx = np.full((nqb, width), -7)
        for b in range(nqb):
            idx[b, :num[b]] = rng.permutation(nkb)[:num[b]]
        vis = O.block_visibility(num, idx, bq, bk, Tq, Tk)
        for i in range(Tq):
            for j in range(Tk):
                listed = [int(x) for x in idx[i // bq, :num[i // bq]]]
                assert vis[i, j] == ((j // bk) in listed), (trial, i, j)


def test_block_visibility_rejects_bad_lists():
    with pytest.raises(ValueError):
        O.block_visibility([1, 1], [[0], [0]], 4, 4, 12, 8)      # three q blocks, two counts
    with pytest.raises(ValueError):
        O.block_visibility([2], [[0, 0]], 4, 4, 4, 8)            # listed twice
    with pytest.raises(ValueError):
        O.block_visibility([1], [[2]], 4, 4, 4, 8)               # index past the last k block


@pytest.mark.parametrize("cap", [0.0, 2.5])
def test_masked_attention_matches_sdpa_bool_mask(cap):
    """Explicit-mask forward against torch SDPA with a boolean mask (rows that
    see nothing excluded: SDPA gives NaN there, the oracle 0 and -inf)."""
    rng = np.random.default_rng(51)
    Tq, Tk, hq, hkv, d = 33, 45, 4, 2, 8
    vis = rng.random((Tq, Tk)) < 0.3
    vis[5] = False
    q, k, v = _rand((Tq, hq, d), rng), _rand((Tk, hkv, d), rng), _rand((Tk, hkv, d), rng)
    out, lse = O.attention_fwd_masked(q, k, v, vis, 0.4, softcap=cap)
    assert np.all(out[5] == 0.0) and np.all(np.isneginf(lse[5]))
    kr, vr = np.repeat(k, hq // hkv, axis=1), np.repeat(v, hq // hkv, axis=1)
    live = vis.any(axis=1)
    if cap == 0:
        ref = _sdpa(q, kr, vr, 0.4, mask=torch.from_numpy(vis))
        np.testing.assert_allclose(out[live], ref[live], rtol=1e-10, atol=1e-12)
    u = 0.4 * np.einsum("ihc,jhc->hij", q, kr)
    s = cap * np.tanh(u / cap) if cap else u
    s = np.where(vis[None], s, -np.inf)
    np.testing.assert_allclose(lse[live], logsumexp(s, axis=-1).T[live], rtol=1e-12, atol=1e-12)


def test_masked_attention_agrees_with_slices():
    """The slice forward and the explicit-mask forward on the slices' mask."""
    rng = np.random.default_rng(52)
    T, d = 70, 8
    qr, kr, ty = W.random_slices(rng, T, T, max_slices=5)
    q, k, v = _rand((T, 2, d), rng), _rand((T, 1, d), rng), _rand((T, 1, d), rng)
    vis = O.visibility(O.normalise_slices(qr, kr, ty, T, T), np.arange(T), np.arange(T)) > 0
    a = O.attention_fwd(q, k, v, qr, kr, ty, 0.3, softcap=1.5)
    b = O.attention_fwd_masked(q, k, v, vis, 0.3, softcap=1.5)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-12, atol=1e-13)


def test_block_slices_plain_cover_the_blocks():
    rng = np.random.default_rng(53)
    Tq, Tk, bq, bk = 37, 29, 8, 6
    nqb, nkb = -(-Tq // bq), -(-Tk // bk)
    num = rng.integers(0, nkb + 1, nqb)
    idx = np.stack([rng.permutation(nkb) for _ in range(nqb)])
    qr, kr, ty = O.block_slices_plain(num, idx, bq, bk, Tq, Tk)
    M = O.visibility(O.normalise_slices(qr, kr, ty, Tq, Tk), np.arange(Tq), np.arange(Tk))
    assert M.max() <= 1
    assert np.array_equal(M > 0, O.block_visibility(num, idx, bq, bk, Tq, Tk))
