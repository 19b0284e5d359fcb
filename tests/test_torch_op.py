"""Custom-operator registration (CPU side): kernels registered, fake shapes, tracing.

The real operators run only on the GPU (tests/test_gpu_compile.py); here the
fake implementations are exercised on fake CUDA tensors, which need no device.
"""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

import range_masked_attention_amd as ffa
from range_masked_attention_amd import torch_op  # noqa: F401


@pytest.mark.parametrize("name", ["ffa_amd::fwd", "ffa_amd::bwd"])
def test_registered(name):
    for key in ("CUDA", "Meta"):
        assert torch._C._dispatch_has_kernel_for_dispatch_key(name, key), (name, key)


def test_fwd_autograd_registered():
    assert torch._C._dispatch_has_kernel_for_dispatch_key("ffa_amd::fwd", "Autograd")


def _fake_inputs(Tq=100, Tk=70, hq=8, hkv=2, d=128, R=5):
    q = torch.empty(Tq, hq, d, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(Tk, hkv, d, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(Tk, hkv, d, dtype=torch.bfloat16, device="cuda")
    qr = torch.zeros(R, 2, dtype=torch.int32, device="cuda")
    kr = torch.zeros(R, 2, dtype=torch.int32, device="cuda")
    ty = torch.zeros(R, dtype=torch.int32, device="cuda")
    return q, k, v, qr, kr, ty


def test_fake_shapes():
    with FakeTensorMode():
        q, k, v, qr, kr, ty = _fake_inputs()
        out, lse, lo = torch.ops.ffa_amd.fwd(q, k, v, qr, kr, ty, 0.1, 0.0)
        assert out.shape == q.shape and out.dtype == torch.bfloat16 and out.device == q.device
        assert lse.shape == (100, 8) and lse.dtype == torch.float32
        assert lo.numel() == 0
        out, lse, lo = torch.ops.ffa_amd.fwd(q, k, v, qr, kr, ty, 0.1, 0.0, None, True)
        assert lo.shape == (ffa.ffa_saved_size(100, 70, 8, 2, 128),) and lo.dtype == torch.uint8
        dq, dk, dv = torch.ops.ffa_amd.bwd(out, q, k, v, out, lse, lo, qr, kr, ty, 0.1, 0.0)
        assert (dq.shape, dk.shape, dv.shape) == (q.shape, k.shape, v.shape)
        assert dq.dtype == dk.dtype == dv.dtype == torch.bfloat16


def test_traces_as_one_opaque_op():
    """make_fx with fake tensors records the operator without running it."""
    def f(q, k, v, qr, kr, ty):
        out, lse = ffa.flex_flash_attn_func(q, k, v, qr, kr, ty, softmax_scale=0.125)
        return out, lse

    with FakeTensorMode():
        args = _fake_inputs(R=7)
    gm = make_fx(f, tracing_mode="fake")(*args)
    targets = [str(n.target) for n in gm.graph.nodes if n.op == "call_function"]
    assert any("ffa_amd.fwd" in t for t in targets), targets


def test_alibi_slopes_argument_is_optional_tensor():
    schema = str(torch.ops.ffa_amd.fwd.default._schema)
    assert "Tensor? alibi_slopes=None" in schema, schema
    assert "Tensor? alibi_slopes=None" in str(torch.ops.ffa_amd.bwd.default._schema)
    with FakeTensorMode():
        q, k, v, qr, kr, ty = _fake_inputs()
        slopes = torch.empty(8, dtype=torch.float32, device="cuda")
        out, lse, _ = torch.ops.ffa_amd.fwd(q, k, v, qr, kr, ty, 0.1, 0.0, slopes)
        assert out.shape == q.shape and lse.shape == (100, 8)


def test_alibi_geometric_slopes():
    # ALiBi's slopes for 8 heads: 1/2, 1/4, ..., 1/256
    assert ffa.alibi_geometric_slopes(8) == [2.0 ** -(h + 1) for h in range(8)]
    s = ffa.alibi_geometric_slopes(32)
    assert len(s) == 32 and all(a > b > 0 for a, b in zip(s, s[1:])) and s[-1] == 2.0 ** -8
