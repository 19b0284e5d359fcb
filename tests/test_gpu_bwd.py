"""Backward parity: ffa_bwd (through the C ABI) against the fp64 oracle.

Small problems are compared over every element of dq, dk, dv.  At full size,
dq is compared on sampled rows, dk and dv on keys near the ends of their
ranges and on keys that the longest lists reach (document starts, the global
sink, window starts; the oracle then computes one kv head), and two exact
identities are checked over all keys:
  sum_j dV_j = sum over rows that see any key of dO_i   (rows of P sum to 1)
  sum_j dK_j = 0 without softcap                        (softmax ignores a
                                                         shift of every key)
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import O, check_grad, dev, ffa, say, to64

pytestmark = pytest.mark.gpu


def _bwd_gpu(q, k, v, do, qr, kr, ty, scale, cap, d, train=True):
    """Forward then backward through the C ABI; with `train` the training
    forward saves its record and the backward takes it (ffa_*_ex), else the
    plain entry points (the backward re-runs the training forward for it)."""
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    if train:
        out, lse, rec = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, cap, train=True)
        dq, dk, dv = ffa.ffa_bwd(qd, kd, vd, out, lse, od, qr, kr, ty, scale, cap, saved=rec)
    else:
        out, lse = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, cap)
        dq, dk, dv = ffa.ffa_bwd(qd, kd, vd, out, lse, od, qr, kr, ty, scale, cap)
    torch.cuda.synchronize()
    return dq, dk, dv


def _cmp(name, got, ref, ctx, mag):
    """Element-wise plain gate (2e-2, plus bf16 half-ulp where |ref| >= 4); returns the max-abs error."""
    return check_grad(name, got, ref, ctx, mag)


def test_pages_shaped_full_compare():
    w = W.config(2)
    say("bwd full compare config 2")
    q, k, v, do = W.workload_tensors(w)
    qr, kr, ty = w.slices()
    dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, w.scale, 0.0, dev())
    rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, w.scale,
                                       magnitudes=True)
    e = [_cmp(n, g, r, "config 2", m) for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags)]
    say(f"  dq/dk/dv max-abs {e[0]:.3e} {e[1]:.3e} {e[2]:.3e}")


CASES = [
    (300, 300, 2, 1, 64, 0.0, 0),
    (257, 190, 4, 2, 128, 0.0, 1),
    (520, 700, 4, 4, 128, 30.0, 2),
    (129, 65, 8, 1, 64, 5.0, 3),
    (700, 500, 2, 2, 128, 0.0, 4),
    (1, 1, 1, 1, 128, 0.0, 6),
    (3, 700, 2, 1, 64, 2.0, 7),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}x{c[1]}_h{c[2]}:{c[3]}_d{c[4]}_cap{c[5]}" for c in CASES])
def test_random_slices_full_compare(case):
    Tq, Tk, hq, hkv, dd, cap, seed = case
    say(f"bwd random slices {case}")
    rng = np.random.default_rng(seed + 50)
    for trial in range(2):
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=2)
        q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, dd, seed=seed * 10 + trial)
        scale = float(rng.uniform(0.05, 0.3))
        dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, cap, dev())
        rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, scale, cap,
                                           magnitudes=True)
        for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags):
            _cmp(n, g, r, f"{case} trial {trial}", m)


def _sink_slices(T, blk, sink, window):
    """Blocks of `blk` rows: each sees keys [0, sink) (FULL) and a causal window."""
    qr, kr, ty = [], [], []
    for b in range(T // blk):
        s, e = b * blk, (b + 1) * blk
        if b == 0:
            qr.append((s, e)); kr.append((0, e)); ty.append(O.CAUSAL)
            continue
        qr.append((s, e)); kr.append((0, sink)); ty.append(O.FULL)
        qr.append((s, e)); kr.append((max(sink, e - window), e)); ty.append(O.CAUSAL)
    return (np.array(qr, np.int32), np.array(kr, np.int32), np.array(ty, np.int32))


# Tiles whose lists are cut into several runs (partial sums added by a
# separate pass).  "sink": the 128-key sink tile is seen by all 64 q tiles
# and is cut into 8 runs, most window tiles into 2.  "cap": 40 key tiles x 8 kv
# heads, each seen by 64 q tiles: runs of 40 entries would need 640 partial
# buffers, over the 512 the workspace holds, so the run length doubles and no
# tile is split (the run-length rule's fallback).
SPLIT_CASES = [
    ("sink", 4096, 4096, 4, 1, 64, 0.0),
    ("sink", 4096, 4096, 8, 2, 128, 30.0),
    ("cap", 4096, 5120, 8, 8, 64, 0.0),
    # a short query block against a long context: each q tile's dQ list is
    # 256 key tiles, cut into 4 runs whose fp32 dQ are added in run order
    ("context", 256, 16384, 4, 1, 128, 0.0),
    ("context", 200, 12000, 2, 2, 64, 15.0),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"{c[0]}_h{c[3]}:{c[4]}_d{c[5]}_cap{c[6]}" for c in SPLIT_CASES])
def test_split_key_tiles_full_compare(case):
    kind, Tq, Tk, hq, hkv, dd, cap = case
    say(f"bwd split key tiles {case}")
    if kind == "sink":
        qr, kr, ty = _sink_slices(Tq, 512, 128, 1024)
    elif kind == "context":
        qr, kr, ty = (np.array([[0, Tq]], np.int32), np.array([[0, Tk]], np.int32), np.array([O.FULL], np.int32))
    else:
        qr, kr, ty = (np.array([[0, Tq]], np.int32), np.array([[0, Tk]], np.int32), np.array([O.FULL], np.int32))
    q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, dd, seed=11)
    scale = dd ** -0.5
    dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, cap, dev())
    again = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, cap, dev())
    for n, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), again):
        assert torch.equal(a, b), f"{case}: {n} differs between two identical calls"
    rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, scale, cap,
                                       magnitudes=True)
    e = [_cmp(n, g, r, str(case), m) for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags)]
    say(f"  dq/dk/dv max-abs {e[0]:.3e} {e[1]:.3e} {e[2]:.3e}")


def _visible_rows(qr, kr, ty, Tq, Tk):
    """Rows that see at least one key (slices are disjoint rectangles)."""
    sl = O.normalise_slices(qr, kr, ty, Tq, Tk)
    sees = np.zeros(Tq, dtype=bool)
    for s in sl:
        _, qs, qe, ks, ke, t = s
        rows = np.arange(qs, qe)
        if t == O.CAUSAL:
            rows = rows[rows - (qe - ke) >= ks]  # row i sees key ks iff ks - ke <= i - qe
        sees[rows] = True
    return sees


@pytest.mark.parametrize("n", [4, 5])
def test_full_size_sampled(n):
    w = W.config(n)
    say(f"bwd full size config {n} ({w.name})")
    q, k, v, do = W.workload_tensors(w)
    qr, kr, ty = w.slices()
    d = dev()
    dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, w.scale, w.softcap, d)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()

    # identities over every key, per kv head
    sees = torch.from_numpy(_visible_rows(qr, kr, ty, w.Tq, w.Tk))
    grp = w.hq // w.hkv
    do_sum = (do.double()[sees].sum(0)).view(w.hkv, grp, w.d).sum(1)
    dv_d = dv.double().cpu()
    dv_sum = dv_d.sum(0)
    bound = 6 * 2.0 ** -8 * dv_d.pow(2).sum(0).sqrt() + 1e-3
    assert torch.all((dv_sum - do_sum).abs() <= bound), float((dv_sum - do_sum).abs().max())
    if w.softcap == 0:
        dk_d = dk.double().cpu()
        kb = 6 * 2.0 ** -8 * dk_d.pow(2).sum(0).sqrt() + 1e-3
        assert torch.all(dk_d.sum(0).abs() <= kb), float(dk_d.sum(0).abs().max())

    # sampled rows of dq and keys of dk/dv, in local clusters so that every
    # oracle block sees only one document's (or window's) columns
    rng = np.random.default_rng(n)
    if n == 4:
        clusters = []
        for b in (2, 7):
            s0, e0 = 8192 * b, 8192 * (b + 1)
            rows = np.unique(np.concatenate([rng.integers(s0, e0, 16), [s0, s0 + 127, s0 + 128, e0 - 1]]))
            keys = np.array([e0 - 130, e0 - 65, e0 - 64, e0 - 2, e0 - 1])
            clusters.append((rows, keys))
    else:
        e0 = w.Tk
        rows = np.unique(np.concatenate([rng.integers(e0 - 1024, e0, 16), [e0 - 1024, e0 - 897, e0 - 1]]))
        keys = np.array([e0 - 130, e0 - 65, e0 - 64, e0 - 2, e0 - 1])
        rows2 = np.unique(np.concatenate([rng.integers(1024, 2048, 8), [1024, 1151, 1152]]))
        clusters = [(rows, keys), (rows2, keys)]
    worst = [0.0, 0.0, 0.0]
    for rows, keys in clusters:
        rq, rk, rv, (mq, mk, mv) = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty,
                                                   w.scale, w.softcap, rows=rows, keys=keys,
                                                   magnitudes=True)
        e = [_cmp("dq", dq[rows], rq, f"config {n}", mq), _cmp("dk", dk[keys], rk, f"config {n}", mk),
             _cmp("dv", dv[keys], rv, f"config {n}", mv)]
        worst = [max(a, b) for a, b in zip(worst, e)]
        say(f"  cluster {len(rows)} rows / {len(keys)} keys: dq/dk/dv max-abs {e[0]:.3e} {e[1]:.3e} {e[2]:.3e}")


# Keys that long q-tile lists reach, where most of the dK/dV work is: the
# first keys of a 8192-token document (seen by all its 8192 rows) on the
# long packed batch, and on the mixed workload the global sink keys (seen by
# all 32768 rows; their key tiles are split into runs whose fp32 partial
# sums are added by a second pass) and window-start keys (seen by four
# 1024-row blocks).  The sink and sliding window are the block-sparse masks
# of the FlexAttention paper summary, section 4.  The oracle computes one kv
# head and the q heads that read it (every one of them, so dk and dv of that
# kv head are complete).
LONG_LIST_CASES = [
    (4, 5, [8192 * 3 + x for x in (0, 1, 63, 64, 127, 128, 4095)]),
    (4, 0, [0, 1, 64, 129]),
    (5, 2, [0, 1, 127, 128, 255, 256, 511, 3072, 3073, 3199, 3200, 20480]),
]


@pytest.mark.parametrize("case", LONG_LIST_CASES, ids=[f"config{c[0]}_kv{c[1]}" for c in LONG_LIST_CASES])
def test_full_size_long_list_keys(case):
    n, g, keys = case
    w = W.config(n)
    say(f"bwd full size long-list keys config {n} kv head {g}: {keys}")
    q, k, v, do = W.workload_tensors(w)
    qr, kr, ty = w.slices()
    dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, w.scale, w.softcap, dev())
    keys = np.array(keys)
    rng = np.random.default_rng(100 + n)
    rows = np.unique(np.concatenate([rng.integers(0, w.Tq, 8), [keys[0], keys[-1]]]))
    grp = w.hq // w.hkv
    heads = list(range(g * grp, (g + 1) * grp))
    rq, rk, rv = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, w.scale, w.softcap,
                                 rows=rows, keys=keys, kv_heads=[g])
    ctx = f"config {n} kv head {g}"
    e = [_cmp("dq", dq[rows][:, heads], rq, ctx, None), _cmp("dk", dk[keys][:, [g]], rk, ctx, None),
         _cmp("dv", dv[keys][:, [g]], rv, ctx, None)]
    say(f"  {len(keys)} keys, {len(rows)} rows: dq/dk/dv max-abs {e[0]:.3e} {e[1]:.3e} {e[2]:.3e}")


@pytest.mark.parametrize("case", [("config2", 0.0), ("sink", 30.0)])
def test_plain_entry_points_rerun_the_forward_bitwise(case):
    """ffa_bwd without a saved record re-runs the training forward to get
    one: the same bits as the training path, split runs included."""
    name, cap = case
    say(f"bwd plain vs training path bitwise ({name})")
    if name == "config2":
        w = W.config(2)
        q, k, v, do = W.workload_tensors(w)
        qr, kr, ty = w.slices()
        scale = w.scale
    else:
        q, k, v, do = W.make_tensors(4096, 4096, 8, 2, 128, seed=12)
        qr, kr, ty = _sink_slices(4096, 512, 128, 1024)
        scale = 128 ** -0.5
    a = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, cap, dev(), train=True)
    b = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, cap, dev(), train=False)
    for n, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), n


def test_operand_range_scaling_is_exact():
    """The fp16 operand copies are scaled by powers of two that map each
    tensor's range onto fp16's, so scaling v by 2^12, dO by 2^-30, q by 2^9
    and k by 2^-9 (far outside fp16's range for dO, near its top for v)
    scales the gradients by exact powers of two, bit for bit:
      dv -> 2^-30 dv,  dq -> 2^(12-30-9) dq,  dk -> 2^(12-30+9) dk.
    (v's copy takes scale 1 inside [2^-3, 16), where a value under 2^-17
    would round in fp16's subnormal range, so v here holds none: its values
    under 2^-8 are zeroed.)"""
    say("bwd range scaling exact")
    Tq, Tk, hq, hkv, dd = 700, 500, 4, 2, 128
    rng = np.random.default_rng(5)
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=2)
    q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, dd, seed=77)
    v = torch.where(v.float().abs() < 2.0 ** -8, torch.zeros_like(v), v)
    scale = 0.11
    base = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, 0.0, dev())
    sq, sk, sv, sd = 2.0 ** 9, 2.0 ** -9, 2.0 ** 12, 2.0 ** -30
    bf = torch.bfloat16
    scaled = _bwd_gpu((q.float() * sq).to(bf), (k.float() * sk).to(bf), (v.float() * sv).to(bf),
                      (do.float() * sd).to(bf), qr, kr, ty, scale, 0.0, dev())
    for n, x, y, f in zip(("dq", "dk", "dv"), base, scaled, (sv * sd * sk, sv * sd * sq, sd)):
        assert torch.equal((x.float() * f).to(bf), y), n


def test_dummy_padding_and_determinism_bitwise():
    """The repro script compares padded and unpadded backward passes (it printed
    ~0.7% max rel diff); this backward is order-free, so they agree bitwise."""
    w = W.config(2)
    say("bwd dummy padding bitwise (config 2)")
    q, k, v, do = W.workload_tensors(w)
    d = dev()
    a = _bwd_gpu(q, k, v, do, *w.slices(padded=False), w.scale, 0.0, d)
    b = _bwd_gpu(q, k, v, do, *w.slices(padded=True), w.scale, 0.0, d)
    c = _bwd_gpu(q, k, v, do, *w.slices(padded=True), w.scale, 0.0, d)
    for x, y, z in zip(a, b, c):
        assert torch.equal(x, y) and torch.equal(y, z)


def test_autograd_through_flex_flash_attn_func():
    w = W.config(1)
    say("autograd through flex_flash_attn_func")
    q, k, v, do = W.workload_tensors(w, with_dout=True)
    d = dev()
    qd, kd, vd = (t.to(d).requires_grad_() for t in (q, k, v))
    qr, kr, ty = w.slices()
    out, lse = ffa.flex_flash_attn_func(qd, kd, vd, qr, kr, ty, softmax_scale=None, softcap=0.0)
    out.backward(do.to(d))
    torch.cuda.synchronize()
    rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, w.scale,
                                       magnitudes=True)
    for (n, g, r), m in zip((("dq", qd.grad, rq), ("dk", kd.grad, rk), ("dv", vd.grad, rv)), mags):
        _cmp(n, g, r, "autograd", m)


def test_plan_reuse_matches_one_shot():
    w = W.config(5)
    say("plan handle reuse (config 5 slices, reduced heads)")
    q, k, v, do = W.make_tensors(w.Tq, w.Tk, 4, 1, 128, seed=3)
    d = dev()
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    qr, kr, ty = w.slices()
    plan = ffa.ffa_plan_create(w.Tq, w.Tk, qr, kr, ty)
    try:
        o1, l1 = ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, w.softcap)
        g1 = ffa.ffa_bwd_planned(plan, qd, kd, vd, o1, l1, od, w.scale, w.softcap)
        o2, l2 = ffa.ffa_fwd_planned(plan, qd, kd, vd, w.scale, w.softcap)
    finally:
        ffa.ffa_plan_destroy(plan)
    o0, l0 = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, w.softcap)
    g0 = ffa.ffa_bwd(qd, kd, vd, o0, l0, od, qr, kr, ty, w.scale, w.softcap)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0) and torch.equal(o2, o0)
    for x, y in zip(g1, g0):
        assert torch.equal(x, y)


def test_guard_band():
    say("bwd guard band")
    Tq, Tk, hq, hkv, dd = 333, 251, 4, 2, 128
    q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, dd, seed=31)
    qr, kr, ty = [[0, 200], [200, 333], [200, 333]], [[0, 251], [0, 30], [40, 251]], [1, 0, 1]
    d = dev()
    G = 4096
    bufs = []

    def guarded(shape, src=None):
        n = int(np.prod(shape))
        buf = torch.full((n + 2 * G,), float("nan"), dtype=torch.bfloat16, device=d)
        view = buf[G:G + n].view(shape)
        if src is not None:
            view.copy_(src.to(d))
        bufs.append(buf)
        return view

    gq, gk, gv, go = guarded(q.shape, q), guarded(k.shape, k), guarded(v.shape, v), guarded(do.shape, do)
    out, lse = ffa.ffa_fwd(gq, gk, gv, qr, kr, ty, 0.09, 0.0)
    n_in = len(bufs)
    gdq, gdk, gdv = guarded(q.shape), guarded(k.shape), guarded(v.shape)
    ffa.ffa_bwd(gq, gk, gv, out, lse, go, qr, kr, ty, 0.09, 0.0, dq=gdq, dk=gdk, dv=gdv)
    ref = _bwd_gpu(q, k, v, do, qr, kr, ty, 0.09, 0.0, d)
    torch.cuda.synchronize()
    for g, r in zip((gdq, gdk, gdv), ref):
        assert torch.equal(g, r)
    for buf in bufs[n_in:]:
        assert torch.isnan(buf[:G].float()).all() and torch.isnan(buf[-G:].float()).all()


# short lists on both sides: key-tile lists of 1 to 5 tiles (dQ walks them)
# and q-tile lists of 1 to 2 tiles (dK/dV walks those, one step per q head),
# ragged last tiles, a causal and a full slice
@pytest.mark.parametrize("Tk", [40, 100, 170, 230, 300])
@pytest.mark.parametrize("causal", [0, 1])
def test_short_lists(Tk, causal):
    say(f"bwd short lists Tk={Tk} causal={causal}")
    Tq, hq, hkv, d = 150, 4, 2, 128
    q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, d, seed=500 + Tk + causal)
    qr = np.array([[0, Tq], [0, 0]], dtype=np.int32)
    kr = np.array([[0, Tk], [0, 0]], dtype=np.int32)
    ty = np.array([causal, 0], dtype=np.int32)
    scale = 0.125
    dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, scale, 0.0, dev())
    rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, scale,
                                       magnitudes=True)
    for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags):
        _cmp(n, g, r, f"Tk {Tk} causal {causal}", m)


# nearly uniform attention (scale 1e-4): every weight within a few ulps of
# 1/l, dV the row average of dO, dq and dk of order the scale
@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_tiny_scale(cap):
    say(f"bwd scale 1e-4 softcap {cap}")
    Tq, Tk, hq, hkv, d = 300, 500, 4, 2, 128
    rng = np.random.default_rng(78)
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=5, n_dummies=1)
    q, k, v, do = W.make_tensors(Tq, Tk, hq, hkv, d, seed=78)
    dq, dk, dv = _bwd_gpu(q, k, v, do, qr, kr, ty, 1e-4, cap, dev())
    rq, rk, rv, mags = O.attention_bwd(to64(q), to64(k), to64(v), to64(do), qr, kr, ty, 1e-4, cap,
                                       magnitudes=True)
    for (n, g, r), m in zip((("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)), mags):
        _cmp(n, g, r, f"scale 1e-4 cap {cap}", m)
