"""GPU parity of attention with a value head dim of its own (attn_fwd_dv):
the HIP path against oracle.attn_fwd_dv on every element, at the fp32 bounds
(|dO| <= 2e-5, |dL| <= 1e-5) and, for 16-bit inputs, at the bf16 / fp16
bounds with the oracle on the rounded inputs. The shapes span several key tiles with
ragged tails and the three key-split settings of the fp32 kernel (problems
with few, some and many 32-row blocks)."""
import numpy as np
import pytest
import torch

import oracle
import scaled_dot_product_12_amd as attn
from scaled_dot_product_12_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
PAIRS = [(128, 64), (64, 128), (16, 32), (32, 16), (128, 16), (16, 128)]
SHAPES = [(1, 1, 100, 300), (2, 8, 70, 45), (4, 16, 300, 50), (8, 32, 300, 33)]


def _inputs(B, H, M, N, D, Dv, seed):
    q, k, _ = make_qkv(B, H, M, N, D, "fp32", seed=seed)
    _, _, v = make_qkv(B, H, M, N, Dv, "fp32", seed=seed + 1)
    return q, k, v


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("D,Dv", PAIRS)
@pytest.mark.parametrize("causal", [False, True])
def test_dv_matches_oracle(shape, D, Dv, causal):
    B, H, M, N = shape
    q, k, v = _inputs(B, H, M, N, D, Dv, seed=40 + D + Dv)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    print(f"[dv] shape={shape} D={D} Dv={Dv} causal={causal}", flush=True)
    o, lse = attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, H, M, Dv)
    ro, rl = oracle.attn_fwd_dv(q, k, v, is_causal=causal, scale=scale)
    do = float(np.abs(o.cpu().double().numpy() - ro).max())
    dl = float(np.abs(lse.cpu().double().numpy() - rl).max())
    assert do <= 2e-5 and dl <= 1e-5, (do, dl)


def test_equal_dims_through_dv_entry_is_attn_fwd():
    q, k, v = (t.to(DEV) for t in make_qkv(2, 4, 130, 90, 64, "bf16", seed=47))
    o1, l1 = attn.attn_fwd(q, k, v, is_causal=True)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    st = attn.lib().attn_fwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                                l2.data_ptr(), 2, 4, 130, 90, 64, 64,
                                attn.default_scale(64), 1, attn.MI355_ATTN_BF16,
                                torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1), (1, 2, 1, 130), (1, 1, 257, 64), (2, 1, 33, 7)])
@pytest.mark.parametrize("D,Dv", [(64, 16), (16, 64), (128, 32)])
def test_dv_edge_shapes(shape, D, Dv):
    B, H, M, N = shape
    q, k, v = _inputs(B, H, M, N, D, Dv, seed=70 + M + N)
    for causal in (False, True):
        o, lse = attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=causal, scale=0.3)
        torch.cuda.synchronize()
        ro, rl = oracle.attn_fwd_dv(q, k, v, is_causal=causal, scale=float(np.float32(0.3)))
        assert np.abs(o.cpu().double().numpy() - ro).max() <= 2e-5
        assert np.abs(lse.cpu().double().numpy() - rl).max() <= 1e-5


def test_dv_empty_queries():
    q, k, v = _inputs(1, 2, 1, 9, 32, 64, seed=77)
    o, lse = attn.attn_fwd(q[:, :, :0].contiguous().to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert tuple(o.shape) == (1, 2, 0, 64) and lse.numel() == 0


PAIRS16 = [(a, b) for a in (16, 32, 64, 128) for b in (16, 32, 64, 128) if a != b]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D,Dv", PAIRS16)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(2, 4, 300, 200), (1, 2, 65, 1), (1, 1, 513, 700)])
def test_dv_16bit_matches_oracle(dtype, D, Dv, causal, shape):
    from parity_util import TOL
    B, H, M, N = shape
    q, k, _ = make_qkv(B, H, M, N, D, dtype, seed=80 + D)
    _, _, v = make_qkv(B, H, M, N, Dv, dtype, seed=81 + Dv)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    print(f"[dv16] {dtype} shape={shape} D={D} Dv={Dv} causal={causal}", flush=True)
    o, lse = attn.attn_fwd(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, H, M, Dv) and o.dtype == q.dtype
    ro, rl = oracle.attn_fwd_dv(q, k, v, is_causal=causal, scale=scale)
    to, tl = TOL[dtype]
    assert np.abs(o.float().cpu().double().numpy() - ro).max() <= to
    assert np.abs(lse.cpu().double().numpy() - rl).max() <= tl
