"""Sizes at the ABI's limit: k and v of 2^31 - 8192 elements (4 GB each).

Every byte offset past 2^31 (and the 32-bit range checks of the buffer
loads) is exercised by slices that reach the far end of the key axis.  The
oracle runs on the visible key ranges only, cut out of k and v with the
slices shifted to match: the attention of a row depends on its visible keys
alone, so this is the same computation.  Keys no slice reaches must get
exactly zero dk and dv.
"""
import numpy as np
import pytest
import torch

from gpu_util import O, check_grad, compare_out_lse, dev, ffa, say, to64

pytestmark = pytest.mark.gpu


def test_keys_at_the_element_limit():
    Tk = (1 << 24) - 64          # Tk * hkv * d = 2^31 - 8192
    Tq, hq, hkv, d = 300, 2, 1, 128
    mid = Tk // 2 + 37
    qr = np.array([[0, 128], [128, 300], [5, 5]], np.int32)
    kr = np.array([[Tk - 700, Tk], [mid, mid + 333], [9, 9]], np.int32)
    ty = np.array([ffa.FULL, ffa.CAUSAL, ffa.FULL], np.int32)
    say(f"limits: Tk={Tk} (k, v {Tk * hkv * d} elements), Tq={Tq}")
    dv_ = dev()
    g = torch.Generator(device=dv_).manual_seed(5)
    q = torch.randn(Tq, hq, d, device=dv_, generator=g).to(torch.bfloat16)
    k = torch.randn(Tk, hkv, d, device=dv_, generator=g, dtype=torch.bfloat16)
    v = torch.randn(Tk, hkv, d, device=dv_, generator=g, dtype=torch.bfloat16)
    do = torch.randn(Tq, hq, d, device=dv_, generator=g).to(torch.bfloat16)
    scale = d ** -0.5
    out, lse = ffa.ffa_fwd(q, k, v, qr, kr, ty, scale, 0.0)
    dq, dk, dv = ffa.ffa_bwd(q, k, v, out, lse, do, qr, kr, ty, scale, 0.0)
    torch.cuda.synchronize()

    # the visible key ranges, cut out; slices shifted into the cut-out axis
    spans = [(int(a), int(b)) for a, b in kr if b > a]
    keys = np.concatenate([np.arange(a, b) for a, b in spans])
    kc, vc = k[torch.from_numpy(keys).to(dv_)].cpu(), v[torch.from_numpy(keys).to(dv_)].cpu()
    base, kr_c = 0, kr.copy()
    for r, (a, b) in enumerate(kr.tolist()):
        if b > a:
            kr_c[r] = (base, base + (b - a))
            base += b - a
        else:
            kr_c[r] = (0, 0)
    ref_out, ref_lse = O.attention_fwd(to64(q.cpu()), to64(kc), to64(vc), qr, kr_c, ty, scale)
    e_out, e_lse = compare_out_lse(out.cpu(), lse.cpu(), ref_out, ref_lse, "limits")
    rq, rk, rv, mags = O.attention_bwd(to64(q.cpu()), to64(kc), to64(vc), to64(do.cpu()), qr, kr_c, ty, scale,
                                       magnitudes=True)
    sel = torch.from_numpy(keys).to(dv_)
    for n, got, ref, m in (("dq", dq, rq, mags[0]), ("dk", dk[sel], rk, mags[1]), ("dv", dv[sel], rv, mags[2])):
        check_grad(n, got, ref, "limits", m)
    # every other key: exactly zero gradient
    for t in (dk, dv):
        t[sel] = 0
        assert int(torch.count_nonzero(t)) == 0
    say(f"  out {e_out:.3e} lse {e_lse:.3e}")
