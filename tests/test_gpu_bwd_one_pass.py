"""GPU parity of the one-pass backward (attn_bwd_ws: dQ shares added in a
fixed order across the key workgroups of a head) against the fp64 gradient
oracle, within the bound of bwd_util.py. Against the two-kernel attn_bwd the
results differ only by summation order (each key workgroup walks the query
tiles from its own starting tile, and dQ is summed share by share), so they
agree to a few units in the last place of the 16-bit type. Every run must
leave the kernel's error word at zero (no wait gave up, the workgroups were
spread over the XCDs as the launch assumes)."""
import math

import numpy as np
import pytest
import torch

import scaled_dot_product_12_amd as attn
from scaled_dot_product_12_amd.inputs import make_dout, make_qkv

from bwd_util import check_heads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _scale(D):
    return float(np.float32(1.0 / math.sqrt(D)))


def _run(q, k, v, g, dtype_code, one_pass, work=None):
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
    o, lse = attn.attn_fwd(qd, kd, vd)
    res = attn.attn_bwd(qd, kd, vd, o, lse, gd, one_pass=one_pass, work=work)
    torch.cuda.synchronize()
    return res


def _close(a, b):
    """The two paths' gradients differ by summation order only: within 8
    units of the 16-bit type's last place of the largest element."""
    for name, x, y in zip(("dQ", "dK", "dV"), a, b):
        u = 2.0 ** -11 if x.dtype == torch.float16 else 2.0 ** -8
        scale = max(float(y.abs().max()), 1e-30)
        d = float((x.float() - y.float()).abs().max())
        assert d <= 8 * u * scale, f"{name}: max |one-pass - two-kernel| {d:.3g} (max {scale:.3g})"


def _work_error(work):
    off = attn.attn_bwd_work_error_offset()
    return int(work[off:off + 4].cpu().view(torch.int32)[0])


def _tickets(work):
    """Workgroups that took a ticket in the last one-pass run (the eight
    per-XCD counters at the start of the work area)."""
    return int(work[:32].cpu().view(torch.int32).sum())


def _ran(work, BH, N):
    """The one-pass kernel ran: every head's key workgroups took a ticket,
    plus those of the heads that pad B*H to a multiple of the XCD count."""
    t = -(-N // 256)
    n = _tickets(work)
    return n % t == 0 and BH * t <= n < (BH + 8) * t


# (B, H, M, N): one and several key workgroups (256 keys each), ragged query
# tiles (32 rows) and key tails, B*H a multiple of the XCD count or not
SHAPES = [
    (1, 8, 300, 600),
    (2, 4, 33, 257),
    (1, 8, 512, 256),
    (4, 2, 100, 1000),
    (1, 8, 1, 1),
    (1, 16, 31, 5),
    (1, 3, 300, 700),
    (3, 5, 97, 513),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_one_pass_against_oracle_and_two_pass(hip_lib, shape, dtype):
    B, H, M, N = shape
    seed = 5 * M + N + (1 if dtype == "fp16" else 0)
    q, k, v = make_qkv(B, H, M, N, 128, dtype, seed)
    g = make_dout(B, H, M, 128, dtype, seed)
    code = attn.MI355_ATTN_FP16 if dtype == "fp16" else attn.MI355_ATTN_BF16
    need = attn.attn_bwd_work_bytes(B, H, M, N, 128, False, code)
    assert need > 0
    print(f"[one-pass] {dtype} {shape} work {need} B", flush=True)
    work = torch.zeros(need, dtype=torch.uint8, device=DEV)
    a = _run(q, k, v, g, code, True, work)
    assert _work_error(work) == 0
    assert _ran(work, B * H, N), "the one-pass kernel did not run"
    b = _run(q, k, v, g, code, False)
    _close(a, b)
    heads = [(0, 0), (B - 1, H - 1)]
    check_heads(q, k, v, g, False, _scale(128), heads=heads, label=f"one-pass-{dtype}")


def test_one_pass_deterministic(hip_lib):
    """Two calls (with a work area that held another call's sums) give the
    same bits."""
    B, H, M, N = 2, 8, 700, 900
    q, k, v = make_qkv(B, H, M, N, 128, "bf16", 61)
    g = make_dout(B, H, M, 128, "bf16", 61)
    need = attn.attn_bwd_work_bytes(B, H, M, N, 128, False, attn.MI355_ATTN_BF16)
    work = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)
    r1 = _run(q, k, v, g, attn.MI355_ATTN_BF16, True, work)
    assert _work_error(work) == 0
    r2 = _run(q, k, v, g, attn.MI355_ATTN_BF16, True, work)
    assert _work_error(work) == 0
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


def test_one_pass_falls_back_where_it_does_not_apply(hip_lib):
    """Causal or D = 64: no work area is needed and the call is attn_bwd."""
    code = attn.MI355_ATTN_BF16
    assert attn.attn_bwd_work_bytes(1, 8, 100, 100, 128, True, code) == 0
    assert attn.attn_bwd_work_bytes(1, 8, 100, 100, 64, False, code) == 0
    q, k, v = make_qkv(1, 6, 100, 130, 64, "bf16", 62)
    g = make_dout(1, 6, 100, 64, "bf16", 62)
    a = _run(q, k, v, g, code, True)
    b = _run(q, k, v, g, code, False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_one_pass_c4_shape(hip_lib):
    """bf16 B=4 H=16 M=N=4096 D=128 through the one-pass path (the launch the
    benchmark times): close to attn_bwd's, two whole heads against the
    oracle."""
    q, k, v = make_qkv(4, 16, 4096, 4096, 128, "bf16", 4)
    g = make_dout(4, 16, 4096, 128, "bf16", 4)
    code = attn.MI355_ATTN_BF16
    work = torch.zeros(attn.attn_bwd_work_bytes(4, 16, 4096, 4096, 128, False, code),
                       dtype=torch.uint8, device=DEV)
    a = _run(q, k, v, g, code, True, work)
    assert _work_error(work) == 0
    assert _ran(work, 4 * 16, 4096), "the one-pass kernel did not run"
    b = _run(q, k, v, g, code, False)
    _close(a, b)
    del a, b
    check_heads(q, k, v, g, False, _scale(128), heads=[(1, 3), (2, 12)], label="c4-one-pass")


def test_one_pass_random_shapes(hip_lib):
    """Seeded random shapes (B*H 1 to 21, so padded heads and not; M up to
    700 and N up to 1300, so one to six key workgroups, with and without the
    rotated tile walk), bf16 and fp16, a work area holding garbage: the
    one-pass kernel runs, leaves its error word at zero, agrees with the
    two-kernel path up to summation order, and one random head of each is
    within the oracle bound."""
    rng = np.random.default_rng(2027)
    for case in range(20):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 8))
        M, N = int(rng.integers(1, 701)), int(rng.integers(1, 1301))
        dtype = "fp16" if case % 3 == 2 else "bf16"
        code = attn.MI355_ATTN_FP16 if dtype == "fp16" else attn.MI355_ATTN_BF16
        seed = 7000 + case
        q, k, v = make_qkv(B, H, M, N, 128, dtype, seed)
        g = make_dout(B, H, M, 128, dtype, seed)
        need = attn.attn_bwd_work_bytes(B, H, M, N, 128, False, code)
        print(f"[one-pass-random] case {case} {dtype} {(B, H, M, N)} work {need} B", flush=True)
        work = torch.full((need,), 0x55, dtype=torch.uint8, device=DEV)
        a = _run(q, k, v, g, code, True, work)
        assert _work_error(work) == 0
        assert _ran(work, B * H, N), "the one-pass kernel did not run"
        b = _run(q, k, v, g, code, False)
        _close(a, b)
        head = (int(rng.integers(0, B)), int(rng.integers(0, H)))
        check_heads(q, k, v, g, False, _scale(128), heads=[head],
                    label=f"one-pass-random-{case}")


def test_one_pass_concurrent_streams(hip_lib):
    """Two one-pass calls in flight at once on two streams, each with its own
    work area, while they share the compute units: no wait gives up, and
    each result equals the same call run alone."""
    code = attn.MI355_ATTN_BF16
    runs = []
    for seed, (B, H, M, N) in ((81, (2, 8, 1024, 1024)), (82, (1, 8, 777, 1500))):
        q, k, v = make_qkv(B, H, M, N, 128, "bf16", seed)
        g = make_dout(B, H, M, 128, "bf16", seed)
        qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, g))
        o, lse = attn.attn_fwd(qd, kd, vd)
        need = attn.attn_bwd_work_bytes(B, H, M, N, 128, False, code)
        runs.append((qd, kd, vd, o, lse, gd, torch.zeros(need, dtype=torch.uint8, device=DEV)))
    torch.cuda.synchronize()
    alone = []
    for (qd, kd, vd, o, lse, gd, work) in runs:
        alone.append(attn.attn_bwd(qd, kd, vd, o, lse, gd, work=work))
        torch.cuda.synchronize()
        assert _work_error(work) == 0
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [None, None]
    print("[one-pass-concurrent] two calls on two streams", flush=True)
    for rep in range(3):
        for i, ((qd, kd, vd, o, lse, gd, work), s) in enumerate(zip(runs, streams)):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                outs[i] = attn.attn_bwd(qd, kd, vd, o, lse, gd, work=work)
        torch.cuda.synchronize()
        for (run, a, b) in zip(runs, outs, alone):
            assert _work_error(run[6]) == 0
            for x, y in zip(a, b):
                assert torch.equal(x, y)
