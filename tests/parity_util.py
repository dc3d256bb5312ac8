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


def check_full_large(q, k, v, causal, scale, label=""):
    """Every element of a large launch against the full oracle, memory-lean:
    the GPU outputs stay fp32 and the comparison runs head by head. Prints
    max|dO| and max|dL|; returns the GPU (O, L) as fp32 / fp64 numpy."""
    import time
    name = dtype_name(q)
    print(f"[parity-full] {label} {name} {tuple(q.shape)} N={k.shape[2]} causal={causal}",
          flush=True)
    dev = torch.device("cuda:0")
    o_d, lse_d = attn.attn_fwd(q.to(dev), k.to(dev), v.to(dev), is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    o = o_d.float().cpu().numpy()
    lse = lse_d.cpu().double().numpy()
    del o_d, lse_d
    t0 = time.perf_counter()
    ro, rl = oracle.attn_fwd(q, k, v, is_causal=causal, scale=scale)
    t_or = time.perf_counter() - t0
    assert np.isfinite(o).all(), "non-finite O"
    assert np.isfinite(lse).all(), "non-finite L"
    do = 0.0
    B, H = q.shape[:2]
    for b in range(B):
        for h in range(H):
            do = max(do, float(np.abs(o[b, h].astype(np.float64) - ro[b, h]).max(initial=0.0)))
    dl = float(np.abs(lse - rl).max(initial=0.0))
    to, tl = TOL[name]
    print(f"[parity-full] {label}: max|dO| = {do:.4g} (<= {to}), max|dL| = {dl:.4g} "
          f"(<= {tl}); oracle {t_or:.1f} s on {oracle.host_threads()} threads", flush=True)
    assert do <= to and dl <= tl, f"{label}: max|dO|={do:.3g} max|dL|={dl:.3g}"
    return o, lse
