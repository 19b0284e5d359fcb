"""Forward parity: the HIP path (through the C ABI) against the fp64 oracle.

Configurations 1-3 (up to 16384 tokens) are compared element by element over
the whole output; the two largest on sampled rows (the oracle computes those
rows one block at a time) plus properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (LSE_TOL, OUT_TOL, O, compare_out_lse, dev, ffa, run_fwd, sample_rows, say,
                      to64)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 2, 3])
def test_config_full_compare(n):
    w = W.config(n)
    say(f"fwd full compare config {n} ({w.name})")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    qr, kr, ty = w.slices()
    out, lse = run_fwd(q, k, v, qr, kr, ty, w.scale, w.softcap, dev())
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, w.scale, w.softcap)
    e_out, e_lse = compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, f"config {n}")
    say(f"  out max-abs {e_out:.3e}  lse max-abs {e_lse:.3e}")


@pytest.mark.parametrize("n", [4, 5])
def test_config_sampled_rows(n):
    w = W.config(n)
    say(f"fwd sampled-row compare config {n} ({w.name}) at full size")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    qr, kr, ty = w.slices()
    out, lse = run_fwd(q, k, v, qr, kr, ty, w.scale, w.softcap, dev())
    # properties over the whole output: finite, every row of these configs
    # sees a key, and each output row is a convex combination of v rows
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    vmax = v.float().abs().amax().item()
    assert out.float().abs().amax().item() <= vmax + OUT_TOL
    rng = np.random.default_rng(n)
    edges = [int(a) for a in np.asarray(qr)[:, 0]] + [int(b) - 1 for b in np.asarray(qr)[:, 1] if b > 0]
    rows = sample_rows(w.Tq, rng, n=160, extra=tuple(edges))
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, w.scale, w.softcap,
                                       rows=rows)
    e_out, e_lse = compare_out_lse(out[rows].cpu(), lse[rows].cpu(), ref_out, ref_lse, f"config {n}")
    say(f"  {len(rows)} rows: out max-abs {e_out:.3e}  lse max-abs {e_lse:.3e}")


CASES = [
    # (Tq, Tk, hq, hkv, d, softcap, seed): ragged tails, GQA ratios, both head sizes
    (300, 300, 2, 1, 64, 0.0, 0),
    (257, 190, 4, 2, 128, 0.0, 1),
    (520, 700, 4, 4, 128, 30.0, 2),
    (129, 65, 8, 1, 64, 5.0, 3),
    (1000, 1000, 2, 2, 128, 0.0, 4),
    (64, 64, 1, 1, 64, 0.0, 5),
    (1, 1, 1, 1, 128, 0.0, 6),
    (3, 700, 2, 1, 64, 0.0, 7),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}x{c[1]}_h{c[2]}:{c[3]}_d{c[4]}_cap{c[5]}" for c in CASES])
def test_random_slices_full_compare(case):
    Tq, Tk, hq, hkv, d, cap, seed = case
    say(f"fwd random slices {case}")
    rng = np.random.default_rng(seed)
    for trial in range(3):
        qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=2)
        q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=seed * 10 + trial, with_dout=False)
        scale = float(rng.uniform(0.05, 0.3))
        out, lse = run_fwd(q, k, v, qr, kr, ty, scale, cap, dev())
        ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, scale, cap)
        compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, f"{case} trial {trial}")


# with softcap the score tiles of the unbiased forward hold the cap's
# reciprocal, whose masked value is +inf: rows with nothing visible must
# still come out as 0 and -inf
@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_short_key_range_causal_rows_empty(cap):
    say(f"fwd causal slice with Lk < Lq, softcap {cap}")
    q, k, v, _ = W.make_tensors(300, 100, 2, 1, 128, seed=11, with_dout=False)
    qr, kr, ty = [[0, 300]], [[0, 100]], [1]
    out, lse = run_fwd(q, k, v, qr, kr, ty, 0.1, cap, dev())
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, 0.1, cap)
    compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, f"Lk<Lq cap {cap}")
    assert torch.all(lse[:200] == float("-inf")) and torch.all(out[:200] == 0)


@pytest.mark.parametrize("slices", [
    (np.zeros((0, 2)), np.zeros((0, 2)), np.zeros(0)),
    (np.zeros((5, 2)), np.zeros((5, 2)), np.ones(5)),
    ([[7, 7], [0, 300]], [[0, 300], [9, 9]], [0, 1]),
], ids=["no_slices", "all_dummies", "both_dummy_kinds"])
def test_nothing_visible(slices):
    say(f"fwd nothing visible")
    q, k, v, _ = W.make_tensors(300, 300, 2, 1, 64, seed=12, with_dout=False)
    d = dev()
    out = torch.full((300, 2, 64), 7.0, dtype=torch.bfloat16, device=d)
    lse = torch.full((300, 2), 7.0, dtype=torch.float32, device=d)
    ffa.ffa_fwd(q.to(d), k.to(d), v.to(d), *slices, 0.1, 0.0, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(lse == float("-inf"))


def test_dummy_padding_bitwise():
    """The repro script's check: padded (R_max=20) vs unpadded slices, 0.0 max rel diff."""
    w = W.config(2)
    say("fwd dummy padding bitwise (config 2)")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    d = dev()
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    o0, l0 = ffa.ffa_fwd(qd, kd, vd, *w.slices(padded=False), w.scale, 0.0)
    o1, l1 = ffa.ffa_fwd(qd, kd, vd, *w.slices(padded=True), w.scale, 0.0)
    # dummies in front, either kind, and the real slices swapped
    qr, kr, ty = w.slices(padded=False)
    qx = np.concatenate([[[5, 5], [0, 2048]], qr[::-1]])
    kx = np.concatenate([[[0, 2048], [100, 100]], kr[::-1]])
    tx = np.concatenate([[1, 0], ty[::-1]])
    o2, l2 = ffa.ffa_fwd(qd, kd, vd, qx, kx, tx, w.scale, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert torch.equal(o0, o2) and torch.equal(l0, l2)


def test_training_forward_record():
    """The training forward (saved record) runs the plain forward's kernel:
    out and lse keep their bits, and the record holds the ranges of q and v,
    out's rounding residual (at most half an ulp of out, with out + residual
    closer to the oracle) and v's fp16 copy."""
    w = W.config(2)
    say("fwd training record (config 2)")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    d = dev()
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    qr, kr, ty = w.slices()
    o0, l0 = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, 0.0)
    o1, l1, rec = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, w.scale, 0.0, train=True)
    torch.cuda.synchronize()
    assert torch.equal(l0, l1) and torch.equal(o0, o1)
    n = o1.numel()
    res = rec[256:256 + 2 * n].view(torch.bfloat16).view(o1.shape)
    ref, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, w.scale)
    compare_out_lse(o1.cpu(), l1.cpu(), ref, ref_lse, "training forward")
    o, r = o1.double().cpu().numpy(), res.double().cpu().numpy()
    # half an ulp of a bf16 value x is 2^(floor(log2 |x|) - 8)
    half_ulp = np.where(o != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(o != 0, o, 1.0)))) - 8), 0.0)
    assert np.all(np.abs(r) <= half_ulp)
    e_train = np.abs(o - ref).max()
    e_full = np.abs(o + r - ref).max()
    say(f"  out max-abs {e_train:.3e}, with the residual {e_full:.3e}")
    assert e_full < e_train
    # the record's range words: max |q| (word 0, left by the forward's waves
    # for the backward's copy of q) and max |v| (word 2), as fp32 bits; the
    # other two are 0
    words = rec[:16].view(torch.int32).cpu()
    want = torch.tensor([float(q.float().abs().max()), 0.0, float(v.float().abs().max()), 0.0]).view(torch.int32)
    assert torch.equal(words, want), (words, want)
    # v's copy: fp16 of v times a power of two s, exact where |s v| is at
    # least 2^-14 (fp16's normal range), else within fp16's subnormal half
    # spacing 2^-25
    kv = v.numel()
    off = 256 + ((2 * n + 255) // 256) * 256
    v16 = rec[off:off + 2 * kv].view(torch.float16).double().cpu().flatten()
    vf = v.double().flatten()
    big = vf.abs() >= 0.125
    ratio = v16[big] / vf[big]
    s = float(ratio[0])
    assert torch.all(ratio == s) and np.log2(s) == round(np.log2(s))
    sv = vf * s
    normal = sv.abs() >= 2.0 ** -14
    assert torch.equal(v16[normal], sv[normal])
    assert float((v16[~normal] - sv[~normal]).abs().max()) <= 2.0 ** -25


def test_v_range_scaling_is_exact():
    """v's fp16 copy is exact at any range: at scale 1 inside [2^-3, 16) and
    at a power of two outside it (a second pass), so scaling v by 2^e scales
    out by 2^e bit for bit and leaves lse alone, on one plan whose room for
    the copy is reused and then grown (d 64, then d 128).  (A value under
    2^-17 at scale 1 falls in fp16's subnormal range and rounds, by less
    than 2^-25, so v here holds none: its values under 2^-8 are zeroed.)"""
    Tq, Tk = 700, 900
    rng = np.random.default_rng(11)
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=6, n_dummies=1)
    d = dev()
    plan = ffa.ffa_plan_create(Tq, Tk, qr, kr, ty)
    try:
        for dd, hq, hkv in ((64, 4, 2), (128, 4, 4)):
            q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, dd, seed=31 + dd, with_dout=False)
            v = torch.where(v.float().abs() < 2.0 ** -8, torch.zeros_like(v), v)
            qd, kd = q.to(d), k.to(d)
            base = None
            for e in (0, 12, -10, 3, -6, 0):
                say(f"fwd v scaled by 2^{e} (d {dd})")
                vd = (v.float() * 2.0 ** e).to(torch.bfloat16).to(d)
                o, l = ffa.ffa_fwd_planned(plan, qd, kd, vd, 0.1, 0.0)
                torch.cuda.synchronize()
                if base is None:
                    base = (o.clone(), l.clone())
                    compare_out_lse(o.cpu(), l.cpu(), *O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, 0.1),
                                    f"v range d {dd}")
                    continue
                assert torch.equal(l, base[1]), e
                assert torch.equal((base[0].float() * 2.0 ** e).to(torch.bfloat16), o), e
    finally:
        ffa.ffa_plan_destroy(plan)
        torch.cuda.synchronize()


def test_run_twice_bitwise():
    w = W.config(3)
    say("fwd determinism (config 3, twice)")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    d = dev()
    qd, kd, vd = q.to(d), k.to(d), v.to(d)
    a = ffa.ffa_fwd(qd, kd, vd, *w.slices(), w.scale, 0.0)
    b = ffa.ffa_fwd(qd, kd, vd, *w.slices(), w.scale, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_guard_band():
    """Tensors inside NaN-filled allocations: no read past the ends leaks in,
    no write lands outside, results match the unguarded run bitwise."""
    say("fwd guard band")
    Tq, Tk, hq, hkv, dd = 333, 251, 4, 2, 128
    q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, dd, seed=21, with_dout=False)
    qr, kr, ty = [[0, 200], [200, 333], [200, 333]], [[0, 251], [0, 30], [40, 251]], [1, 0, 1]
    d = dev()
    G = 4096

    def guarded(t, dtype=torch.bfloat16):
        n = t.numel()
        buf = torch.full((n + 2 * G,), float("nan"), dtype=dtype, device=d)
        view = buf[G:G + n].view(t.shape)
        view.copy_(t.to(d))
        return buf, view

    bq, gq = guarded(q)
    bk, gk = guarded(k)
    bv, gv = guarded(v)
    bo, go = guarded(torch.zeros(Tq, hq, dd))
    bl, gl = guarded(torch.zeros(Tq, hq), torch.float32)
    ffa.ffa_fwd(gq, gk, gv, qr, kr, ty, 0.09, 0.0, out=go, lse=gl)
    ro, rl = ffa.ffa_fwd(q.to(d), k.to(d), v.to(d), qr, kr, ty, 0.09, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(go, ro) and torch.equal(gl, rl)
    for buf in (bo, bl):
        assert torch.isnan(buf[:G].float()).all() and torch.isnan(buf[-G:].float()).all()


def test_flex_flash_attn_func_api():
    """The pages' call shape: slice tensors on the device, max_seqlen args, default scale."""
    w = W.config(2)
    say("flex_flash_attn_func API")
    q, k, v, _ = W.workload_tensors(w, with_dout=False)
    d = dev()
    qr, kr, ty = (torch.from_numpy(x).to(d) for x in w.slices())
    out, lse = ffa.flex_flash_attn_func(q.to(d), k.to(d), v.to(d), qr, kr, ty,
                                        max_seqlen_q=w.Tq, max_seqlen_k=w.Tk,
                                        softmax_scale=None, softcap=0)
    ref, ref_lse = ffa.ffa_fwd(q.to(d), k.to(d), v.to(d), *w.slices(), w.scale, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_invalid_tensor_arguments_raise():
    d = dev()
    q = torch.zeros(16, 2, 64, dtype=torch.bfloat16, device=d)
    with pytest.raises(TypeError):
        ffa.ffa_fwd(q.float(), q, q, [[0, 16]], [[0, 16]], [0], 0.1)
    with pytest.raises(ValueError):
        ffa.ffa_fwd(q.transpose(0, 1), q, q, [[0, 16]], [[0, 16]], [0], 0.1)
    with pytest.raises(ffa.FfaError, match="q range"):
        ffa.ffa_fwd(q, q, q, [[0, 17]], [[0, 16]], [0], 0.1)


# Long q-tile lists cut into runs (of at least 64 key tiles) whose outputs
# are merged by their lse: a short query block against a long context (each
# q tile's list is 512 key tiles: 8 runs per tile), and a causal slice whose
# rows see a long prefix (141 key tiles: 3 runs), with softcap and the
# distance bias (runs walked downwards).
SPLIT_CASES = [
    ("context", 256, 32768, 4, 1, 128, 0.0, False),
    ("prefix", 300, 9000, 2, 2, 64, 20.0, True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_q_tiles_full_compare(case):
    name, Tq, Tk, hq, hkv, d, cap, bias = case
    say(f"fwd split q tiles {case}")
    if name == "context":
        qr, kr, ty = [[0, Tq], [7, 7]], [[0, Tk], [0, 0]], [0, 0]
    else:
        qr, kr, ty = [[0, Tq]], [[0, Tk]], [1]
    q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=21, with_dout=False)
    scale = d ** -0.5
    dv_ = dev()
    slopes = np.array(ffa.alibi_geometric_slopes(hq)) if bias else None
    st = torch.tensor(slopes, dtype=torch.float32, device=dv_) if bias else None
    qd, kd, vd = q.to(dv_), k.to(dv_), v.to(dv_)
    out, lse = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, cap, alibi_slopes=st)
    out2, lse2 = ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, scale, cap, alibi_slopes=st)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    sl32 = st.double().cpu().numpy() if bias else None
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, scale, cap, alibi_slopes=sl32)
    e_out, e_lse = compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, name)
    say(f"  out max-abs {e_out:.3e}  lse max-abs {e_lse:.3e}")


@pytest.mark.parametrize("Tq,Tk", [(300, 0), (0, 300)])
def test_empty_token_axis(Tq, Tk):
    """No keys: every row sees nothing (out 0, lse -inf, dq 0).  No queries:
    every key is seen by nothing (dk = dv = 0)."""
    say(f"empty axis Tq={Tq} Tk={Tk}")
    d = dev()
    q, k, v, do = W.make_tensors(Tq, Tk, 4, 2, 128, seed=13)
    qd, kd, vd, od = q.to(d), k.to(d), v.to(d), do.to(d)
    for qr, kr, ty in (([[0, Tq]], [[0, Tk]], [1]), ([[0, 0], [0, 0]], [[0, 0], [0, 0]], [0, 1]), ([], [], [])):
        out = torch.full_like(qd, 7.0)
        lse = torch.full((Tq, 4), 7.0, dtype=torch.float32, device=d)
        ffa.ffa_fwd(qd, kd, vd, qr, kr, ty, 0.1, 0.0, out=out, lse=lse)
        dq, dk, dv = (torch.full_like(t, 7.0) for t in (qd, kd, vd))
        ffa.ffa_bwd(qd, kd, vd, out, lse, od, qr, kr, ty, 0.1, 0.0, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        assert torch.all(out == 0) and torch.all(lse == float("-inf"))
        assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


# key-tile lists of 1 to 5 tiles (64 keys a tile, ragged last tile), walked
# upwards and, with positive distance-bias slopes, downwards: the forward
# carries the entries of the next positions and prefetches the one after,
# clamped at the end of the list
@pytest.mark.parametrize("Tk", [40, 100, 170, 230, 300])
@pytest.mark.parametrize("walk", ["up", "down"])
def test_short_key_lists(Tk, walk):
    say(f"fwd short key list Tk={Tk} walk={walk}")
    Tq, hq, hkv, d = 200, 4, 2, 128
    q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=Tk, with_dout=False)
    qr = np.array([[0, Tq], [0, 0]], dtype=np.int32)
    kr = np.array([[0, Tk], [0, 0]], dtype=np.int32)
    ty = np.array([0, 0], dtype=np.int32)
    scale = 0.125
    dv_ = dev()
    if walk == "up":
        out, lse = run_fwd(q, k, v, qr, kr, ty, scale, 0.0, dv_)
        slopes = None
    else:
        st = torch.full((hq,), 0.05, dtype=torch.float32, device=dv_)
        out, lse = ffa.ffa_fwd_ex(q.to(dv_), k.to(dv_), v.to(dv_), qr, kr, ty, scale, 0.0, st)
        torch.cuda.synchronize()
        slopes = st.double().cpu().numpy()
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, scale, 0.0, alibi_slopes=slopes)
    compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, f"Tk {Tk} {walk}")


# softmax temperatures far from the workloads' 1/sqrt(d): nearly uniform
# weights (scale 1e-4: every exponent within a few ulps of the max) and
# nearly one-hot rows (scale 3: logits with a spread of hundreds, so the
# running max moves by far more than the lazy-rescale threshold), with and
# without softcap
@pytest.mark.parametrize("scale", [1e-4, 3.0])
@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_extreme_scales(scale, cap):
    say(f"fwd extreme scale {scale} softcap {cap}")
    Tq, Tk, hq, hkv, d = 300, 500, 4, 2, 128
    rng = np.random.default_rng(77)
    qr, kr, ty = W.random_slices(rng, Tq, Tk, max_slices=5, n_dummies=1)
    q, k, v, _ = W.make_tensors(Tq, Tk, hq, hkv, d, seed=77, with_dout=False)
    out, lse = run_fwd(q, k, v, qr, kr, ty, scale, cap, dev())
    ref_out, ref_lse = O.attention_fwd(to64(q), to64(k), to64(v), qr, kr, ty, scale, cap)
    compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, f"scale {scale} cap {cap}")
