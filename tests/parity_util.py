"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same (exact) inputs, compare within the stated tolerances."""
import numpy as np
import torch

import oracle
import scaled_dot_product_12_amd as attn

# max |dO| and max |dL| against the fp64 oracle (the oracle consumes the
# exact fp32 / bf16- / fp16-rounded inputs the GPU sees). fp32 and bf16 are
# the stated bounds. fp16 has none stated: its error has the same sources as
# bf16's (P and O rounded to the input type, everything else fp32), each
# proportional to the unit roundoff, so the bf16 bounds are scaled by
# 2^-11 / 2^-8 = 1/8. The largest |O| of these inputs (< 8) has a half-ulp of
# at most 2^-9 ~ 1.95e-3 in fp16, inside the O bound.
TOL = {"fp32": (2e-5, 1e-5), "bf16": (2e-2, 1e-2), "fp16": (2.5e-3, 1.25e-3)}
TDT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def dtype_name(t):
    return {torch.float32: "fp32", torch.bfloat16: "bf16", torch.float16: "fp16"}[t.dtype]


def run_gpu(q, k, v, causal, scale, path=attn.MI355_ATTN_PATH_AUTO):
    dev = torch.device("cuda:0")
    o, lse = attn.attn_fwd(q.to(dev), k.to(dev), v.to(dev), is_causal=causal,
                           scale=scale, path=path)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def max_err(o, lse, ro, rl):
    assert np.isfinite(o).all(), "non-finite O"
    assert np.isfinite(lse).all(), "non-finite L"
    return float(np.abs(o - ro).max(initial=0.0)), float(np.abs(lse - rl).max(initial=0.0))


def fp32_magnitude_tol(D, rl):
    """Bound for fp32 problems whose scores are far larger than those of the
    workloads (scale well above 1/sqrt(D)): a length-D fp32 dot product with
    fp32 accumulation carries a rounding error of about sqrt(D) * u * |s|
    (u = 2^-24), and L ~ max_j s_j, so the stated absolute bounds are widened
    to 4 * sqrt(D) * u * max|L| when that is larger."""
    return 4.0 * np.sqrt(D) * 2.0 ** -24 * float(np.abs(rl).max(initial=0.0))


def check_full(q, k, v, causal, scale, path=attn.MI355_ATTN_PATH_AUTO, label="",
               magnitude_tol=False):
    """Every output element against the full oracle."""
    name = dtype_name(q)
    print(f"[parity] {label} {name} {tuple(q.shape)} N={k.shape[2]} causal={causal} "
          f"path={path}", flush=True)
    o, lse = run_gpu(q, k, v, causal, scale, path)
    ro, rl = oracle.attn_fwd(q, k, v, is_causal=causal, scale=scale)
    do, dl = max_err(o, lse, ro, rl)
    to, tl = TOL[name]
    if magnitude_tol and name == "fp32":
        extra = fp32_magnitude_tol(q.shape[-1], rl)
        to, tl = max(to, extra), max(tl, extra)
    assert do <= to and dl <= tl, f"{label}: max|dO|={do:.3g} (<= {to}) max|dL|={dl:.3g} (<= {tl})"
    return do, dl


def sample_rows(B, H, M, n_random, seed, tile_edges=(0, 1, 31, 32, 63, 64, 127, 128, 255, 256)):
    """Query rows (b, h, i): tile edges and the last row of a few heads, plus
    seeded random rows anywhere."""
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (B - 1, H - 1), (B // 2, H // 2)}
    rows = set()
    for b, h in heads:
        for i in tile_edges:
            if i < M:
                rows.add((b, h, i))
        for i in (M - 1, M - 2, M // 2):
            if 0 <= i < M:
                rows.add((b, h, i))
    for _ in range(n_random):
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(M))))
    return sorted(rows)


def check_sampled(q, k, v, causal, scale, n_random=300, seed=0, label=""):
    """Full-size launch; the oracle evaluates sampled rows one by one."""
    name = dtype_name(q)
    B, H, M, D = q.shape
    print(f"[parity-sampled] {label} {name} {tuple(q.shape)} N={k.shape[2]} "
          f"causal={causal}", flush=True)
    o, lse = run_gpu(q, k, v, causal, scale)
    rows = sample_rows(B, H, M, n_random, seed)
    ro, rl = oracle.attn_rows(q, k, v, rows, is_causal=causal, scale=scale)
    go = np.stack([o[b, h, i] for b, h, i in rows])
    gl = np.array([lse[b, h, i] for b, h, i in rows])
    do, dl = max_err(go, gl, ro, rl)
    to, tl = TOL[name]
    assert do <= to and dl <= tl, f"{label}: max|dO|={do:.3g} max|dL|={dl:.3g}"
    return o, lse
