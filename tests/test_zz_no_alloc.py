"""attn_bwd_noalloc (delta in the library's static device array, no
allocation) against attn_bwd (delta in a caller workspace; its two-kernel
form, which the no-alloc entry is a variant of): the same kernels, so the
gradients must be bit-identical. Two calls in a row, the second on a
smaller problem (the array keeps the first call's delta; the second must not
depend on it), then a problem above the array's capacity, which is refused
before launching."""
import pytest
import torch

import scaled_dot_product_12_amd as attn
from scaled_dot_product_12_amd.inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _problem(B, H, M, N, D, dtype, causal, seed):
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, M, N, D, dtype, seed))
    g = make_dout(B, H, M, D, dtype, seed).to(DEV)
    o, lse = attn.attn_fwd(q, k, v, is_causal=causal)
    return q, k, v, g, o, lse


def _both(q, k, v, g, o, lse, causal):
    ref = attn.attn_bwd(q, k, v, o, lse, g, is_causal=causal, one_pass=False)
    out = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    got = attn.attn_bwd_noalloc(q, k, v, o, lse, g, out, is_causal=causal)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_backward_equals_workspace_backward(dtype, causal):
    for label, shape in (("large", (2, 4, 700, 650, 128)), ("smaller", (1, 3, 133, 257, 64))):
        print(f"[noalloc] {label} {shape} {dtype} causal={causal}", flush=True)
        B, H, M, N, D = shape
        q, k, v, g, o, lse = _problem(B, H, M, N, D, dtype, causal, seed=M + N)
        ref, got = _both(q, k, v, g, o, lse, causal)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.isfinite(a).all(), (label, name)
            assert torch.equal(a, b), (label, name)


def test_noalloc_rejects_problems_above_the_scratch_capacity():
    cap = attn.MI355_ATTN_NOALLOC_MAX_ROWS
    M = cap // 2 + 1  # B*H*M = cap + 2 with B*H = 2
    q = torch.zeros(1, 2, M, 32, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(1, 2, M, device=DEV)
    out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(k))
    with pytest.raises(RuntimeError, match="scratch"):
        attn.attn_bwd_noalloc(q, k, k, q, lse, q, out)
