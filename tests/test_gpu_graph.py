"""The entry points captured in a HIP graph (as the benchmark times the
microsecond workloads): every replay must reproduce the eager result bit for
bit. Between replays the outputs are overwritten with NaN and unrelated eager
work runs, so a replay that skipped a write or raced would show."""
import pytest
import torch

import scaled_dot_product_12_amd as attn
from scaled_dot_product_12_amd.inputs import make_axial_block, make_qkv

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _replay_matches(launch, outs, replays=3):
    launch()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            launch()
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device=DEV)
    for r in range(replays):
        for t in outs:
            t.fill_(float("nan"))
        noise.mul_(1.0001).add_(1.0)   # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {r} differs from the eager result"


@pytest.mark.parametrize("case", [
    ("fp32", 128, 4, 32, 32, 16, False),   # one axial pass: the short-sequence kernel
    ("fp32", 1, 1, 128, 128, 64, False),   # single head: fp32 main kernel
    ("bf16", 1, 2, 300, 300, 128, True),   # 16-bit main kernel, causal, ragged
])
def test_attn_fwd_graph_replays(case):
    dtype, B, H, M, N, D, causal = case
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, M, N, D, dtype, seed=31))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, M), dtype=torch.float32, device=DEV)
    _replay_matches(lambda: attn.attn_fwd(q, k, v, is_causal=causal, out=(o, lse)), [o, lse])


def test_axial_block_graph_replays():
    x, row, col = make_axial_block(4, 32, 32, 64, seed=32)
    x = x.to(DEV)
    row = tuple(t.to(DEV) for t in row)
    col = tuple(t.to(DEV) for t in col)
    out = torch.empty_like(x)
    _replay_matches(lambda: attn.axial_block(x, row, col, out=out), [out])


@pytest.mark.parametrize("one_pass", [True, False])
def test_attn_bwd_graph_replays(one_pass):
    """The backward in a graph: the one-pass path (delta kernel clearing the
    counters of a preallocated work area, then the fused kernel) and the two
    kernels; the work area keeps the previous replay's sums and counters, and
    every replay must still give the eager gradients."""
    from scaled_dot_product_12_amd.inputs import make_dout
    B, H, M, N, D = 1, 8, 300, 600, 128
    q, k, v = (t.to(DEV) for t in make_qkv(B, H, M, N, D, "bf16", seed=33))
    g = make_dout(B, H, M, D, "bf16", seed=33).to(DEV)
    o, lse = attn.attn_fwd(q, k, v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, H, M), dtype=torch.float32, device=DEV)
    need = attn.attn_bwd_work_bytes(B, H, M, N, D, False, attn.MI355_ATTN_BF16)
    assert need > 0
    work = torch.empty(need, dtype=torch.uint8, device=DEV)
    _replay_matches(lambda: attn.attn_bwd(q, k, v, o, lse, g, out=(dq, dk, dv), delta=delta,
                                          one_pass=one_pass, work=work), [dq, dk, dv])
    off = attn.attn_bwd_work_error_offset()
    assert int(work[off:off + 4].cpu().view(torch.int32)[0]) == 0
