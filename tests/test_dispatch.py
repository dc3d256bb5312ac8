"""The PyTorch-facing layer (scaled_dot_product_12_amd.dispatch): the SDPA
checker's decisions (CPU), and on the GPU that the SDPA drop-in and the
autograd op run exactly the C-ABI kernels (bit-identical results) with
gradients within the derived bound of the oracle."""
import math

import numpy as np
import pytest
import torch

from scaled_dot_product_12_amd.inputs import make_dout, make_qkv


def _dispatch():
    from scaled_dot_product_12_amd import dispatch
    return dispatch


def test_checker_rejections_on_cpu(hip_lib):
    d = _dispatch()
    q = torch.zeros(1, 2, 8, 64)
    ok, why = d.sdpa_checker(q, q, q)
    assert not ok and "GPU" in why
    for kw, word in ((dict(attn_mask=torch.ones(8, 8)), "attn_mask"),
                     (dict(dropout_p=0.1), "dropout"),
                     (dict(enable_gqa=True), "grouped")):
        ok, why = d.sdpa_checker(q, q, q, **kw)
        assert not ok and word in why
    with pytest.raises(NotImplementedError):
        d.scaled_dot_product_attention(q, q, q)


class _SdpaBlock(torch.nn.Module):
    """An attention layer written against torch's own SDPA, as model code is:
    it knows nothing of this library."""

    def __init__(self, causal):
        super().__init__()
        self.causal = causal

    def forward(self, q, k, v):
        return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=self.causal)


def test_route_sdpa_intercepts_torch_sdpa_on_cpu(hip_lib):
    """The mode sees the module's torch SDPA call: strict, the checker's
    reason is raised (CPU tensors are not the library's); non-strict, torch's
    own SDPA runs and gives its usual result. Other torch calls are untouched."""
    d = _dispatch()
    q, k, v = make_qkv(1, 2, 9, 11, 16, "fp32", seed=3)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    blk = _SdpaBlock(causal=True)
    with d.route_sdpa() as mode:
        assert torch.equal(q + 1, q.add(1))
        with pytest.raises(NotImplementedError, match="not on a GPU"):
            blk(q, k, v)
        with pytest.raises(NotImplementedError, match="attn_mask"):
            torch.nn.functional.scaled_dot_product_attention(q, k, v, torch.ones(9, 11) > 0)
    assert mode.routed == 0
    with d.route_sdpa(strict=False) as mode:
        out = blk(q, k, v)
        out2 = torch.nn.functional.scaled_dot_product_attention(q, k, v, None, 0.0, True)
    assert torch.equal(out, ref) and torch.equal(out2, ref)
    assert (mode.routed, mode.declined) == (0, 2)
    with pytest.raises(TypeError):
        with d.route_sdpa():
            torch.nn.functional.scaled_dot_product_attention(q, k, v, bogus=1)




def _gpu(*ts):
    return tuple(t.to("cuda:0") for t in ts)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_sdpa_dropin_is_the_library_forward(hip_lib, dtype, causal):
    d = _dispatch()
    q, k, v = _gpu(*make_qkv(2, 3, 150, 200, 64, dtype, seed=61))
    with torch.no_grad():
        ok, why = d.sdpa_checker(q, k, v, is_causal=causal)
        assert ok, why
        o = d.scaled_dot_product_attention(q, k, v, is_causal=causal)
        ref, _ = hip_lib.attn_fwd(q, k, v, is_causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)


@pytest.mark.gpu
def test_non_contiguous_views(hip_lib):
    """[B, seq, H, D] storage viewed as [B, H, seq, D] (a transpose), the
    common layout of model code: copied to contiguous, same result."""
    d = _dispatch()
    q, k, v = _gpu(*make_qkv(2, 3, 130, 130, 128, "bf16", seed=62))
    qt, kt, vt = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (q, k, v))
    assert not qt.is_contiguous()
    with torch.no_grad():
        a = d.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
        b = d.scaled_dot_product_attention(q, k, v, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_autograd_is_the_library_backward(hip_lib, dtype, causal):
    import oracle
    from bwd_util import U_BF16, U_F16, head_bounds
    d = _dispatch()
    q0, k0, v0 = make_qkv(1, 2, 190, 170, 128, dtype, seed=63)
    g0 = make_dout(1, 2, 190, 128, dtype, seed=63)
    q, k, v = (t.to("cuda:0").requires_grad_(True) for t in (q0, k0, v0))
    g = g0.to("cuda:0")
    o = d.attention(q, k, v, is_causal=causal)
    o.backward(g)
    torch.cuda.synchronize()
    with torch.no_grad():
        ref_o, lse = hip_lib.attn_fwd(q, k, v, is_causal=causal)
        ref = hip_lib.attn_bwd(q.detach(), k.detach(), v.detach(), ref_o, lse, g,
                               is_causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), ref_o)
    for got, r in zip((q.grad, k.grad, v.grad), ref):
        assert torch.equal(got, r)
    scale = float(np.float32(1.0 / math.sqrt(128)))
    refs = oracle.attn_bwd(q0, k0, v0, g0, is_causal=causal, scale=scale)
    for h in range(2):
        f64 = lambda t: t[0, h].double().numpy()
        bounds = head_bounds(f64(q0), f64(k0), f64(v0), f64(g0), scale, causal,
                             tuple(x[0, h] for x in refs), U_F16 if dtype == "fp16" else U_BF16)
        for got, r, bd in zip((q.grad, k.grad, v.grad), refs, bounds):
            err = np.abs(got[0, h].float().cpu().double().numpy() - r[0, h])
            assert (err <= bd).all()


@pytest.mark.gpu
def test_checker_on_gpu_tensors(hip_lib):
    d = _dispatch()
    q, k, v = _gpu(*make_qkv(1, 1, 8, 8, 16, "bf16", seed=64))
    assert d.sdpa_checker(q, k, v)[0]                      # forward only: D = 16 is fine
    q.requires_grad_(True)
    ok, why = d.sdpa_checker(q, k, v)
    assert not ok and "backward" in why                   # no D = 16 backward
    with torch.no_grad():
        assert d.sdpa_checker(q, k, v)[0]                  # no grad needed
    qf, kf, vf = _gpu(*make_qkv(1, 1, 8, 8, 64, "fp32", seed=65))
    qf.requires_grad_(True)
    assert not d.sdpa_checker(qf, kf, vf)[0]               # no fp32 backward
    q16 = qf.detach().half()
    assert d.sdpa_checker(q16, q16, q16)[0]                # fp16 forward
    q16.requires_grad_(True)
    assert d.sdpa_checker(q16, q16.detach(), q16.detach())[0]  # fp16 backward too
    ok, why = d.sdpa_checker(q.detach(), k, v, attn_mask=torch.ones(8, 8, device="cuda:0"))
    assert not ok


@pytest.mark.gpu
def test_sdpa_dropin_value_head_dim_of_its_own(hip_lib):
    """Dv != D runs (attn_fwd_dv, same result as the binding); an unsupported
    Dv and gradient requests are refused with the reason."""
    d = _dispatch()
    q, k, _ = _gpu(*make_qkv(2, 3, 90, 120, 64, "fp32", seed=66))
    (v,) = _gpu(make_qkv(2, 3, 90, 120, 32, "fp32", seed=67)[2])
    with torch.no_grad():
        assert d.sdpa_checker(q, k, v, is_causal=True)[0]
        o = d.scaled_dot_product_attention(q, k, v, is_causal=True)
        ref, _ = hip_lib.attn_fwd(q, k, v, is_causal=True)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (2, 3, 90, 32) and torch.equal(o, ref)
    assert d.sdpa_checker(q.bfloat16(), k.bfloat16(), v.bfloat16())[0]
    ok, why = d.sdpa_checker(q, k, v[..., :24].contiguous())
    assert not ok and "value head dim" in why
    q.requires_grad_(True)
    ok, why = d.sdpa_checker(q, k, v)
    assert not ok and "backward" in why


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "fp32", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_route_sdpa_runs_an_unmodified_module_on_the_library(hip_lib, dtype, causal):
    """A module that calls torch's SDPA, run under route_sdpa: its output is
    bit-equal to attn_fwd's, and (16-bit) its gradients to attn_bwd's."""
    d = _dispatch()
    q0, k0, v0 = make_qkv(2, 4, 300, 257, 128, dtype, seed=68)
    blk = _SdpaBlock(causal)
    q, k, v = _gpu(q0, k0, v0)
    with torch.no_grad():
        ref_o, lse = hip_lib.attn_fwd(q, k, v, is_causal=causal)
        with d.route_sdpa() as mode:
            o = blk(q, k, v)
    torch.cuda.synchronize()
    assert mode.routed == 1 and torch.equal(o, ref_o)
    if dtype == "fp32":
        return
    g = make_dout(2, 4, 300, 128, dtype, seed=68).to("cuda:0")
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    with d.route_sdpa() as mode:
        o = blk(qg, kg, vg)
    o.backward(g)
    with torch.no_grad():
        ref = hip_lib.attn_bwd(q, k, v, ref_o, lse, g, is_causal=causal)
    torch.cuda.synchronize()
    assert mode.routed == 1 and torch.equal(o.detach(), ref_o)
    for got, r in zip((qg.grad, kg.grad, vg.grad), ref):
        assert torch.equal(got, r)
