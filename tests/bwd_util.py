"""Helpers for the backward GPU parity tests: run attn_fwd then attn_bwd on
the GPU, run the fp64 gradient oracle on the same (exact bf16 / fp16) inputs,
and compare every element against a bound derived from the arithmetic.

The bound (unit roundoff u of the 16-bit input type: 2^-8 for bf16, 2^-11 for
fp16; fp32 u32 = 2^-24, lambda = 8):
each gradient element is a sum over n rows of terms a_i, and the kernels
round each term's factor once to the input type (P for dV, dS for dK and dQ) with
errors that are independent between terms, so by Hoeffding's inequality the
sum's error stays below lambda * u * sqrt(sum_i abar_i^2) except with
probability 2 exp(-lambda^2 / 2) ~ 2.5e-14 per element. abar_i is the term's
magnitude with every source of error in it:
    dV_jd:  P_ij |dO_id|
    dK_jd:  scale P_ij (|dP_ij| + |delta_i| + dabs_i) |q_id|
    dQ_id:  scale P_ij (|dP_ij| + |delta_i|) |k_jd|
where dabs_i = sum_d |O_id dO_id| bounds the error of delta_i taken from the
rounded forward output (its own rounding and the forward's error, each
at most u * dabs_i). In dQ that error is common to the whole row, so it is
added coherently: 2 u scale dabs_i sum_j P_ij |k_jd|. fp32 accumulation adds
lambda * sqrt(n) * u32 * sum_i abar_i, and rounding the result to the input type
u * |ref|.

Gradual underflow: below the smallest normal number of the input type
(2^-14 for fp16, 2^-126 for bf16) a rounded value errs by up to half the
subnormal spacing, h = 2^-25 (fp16) or 2^-134 (bf16), not by u times its
magnitude. So each rounded factor errs by at most u |x| + h: the terms add
lambda * h * s * sqrt(sum_i x_i^2) over the terms that are not masked out
(s the factor's multiplier: 1 for P in dV, scale for dS in dK and dQ; x the
other operand), and the rounded result h when it is not an exact zero.
"""
import numpy as np
import torch

import oracle
import scaled_dot_product_12_amd as attn

U_BF16 = 2.0 ** -8
U_F16 = 2.0 ** -11
U_F32 = 2.0 ** -24
# half the subnormal spacing of each 16-bit type
H_BF16 = 2.0 ** -134
H_F16 = 2.0 ** -25
LAMBDA = 8.0


def gpu_fwd_bwd(q, k, v, g, causal, scale, one_pass=True):
    """attn_fwd then attn_bwd on cuda:0; returns numpy fp64 (dq, dk, dv) and
    the GPU (o, lse)."""
    dev = torch.device("cuda:0")
    qd, kd, vd, gd = (t.to(dev) for t in (q, k, v, g))
    o, lse = attn.attn_fwd(qd, kd, vd, is_causal=causal, scale=scale)
    dq, dk, dv = attn.attn_bwd(qd, kd, vd, o, lse, gd, is_causal=causal, scale=scale,
                               one_pass=one_pass)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().double().numpy()
    return f(dq), f(dk), f(dv), o, lse


def head_bounds(q, k, v, g, scale, causal, refs, u=U_BF16):
    """Per-element bounds for one head (2-D fp64 arrays q [M,D], k, v [N,D],
    g [M,D]); refs = oracle (dq, dk, dv) of that head; u = unit roundoff of
    the input type."""
    M, N = q.shape[0], k.shape[0]
    o_ref, l_ref = oracle.attn_fwd(q[None, None], k[None, None], v[None, None],
                                   is_causal=causal, scale=scale)
    O, L = o_ref[0, 0], l_ref[0, 0]
    S = scale * (q @ k.T)
    if causal:
        S = np.where(np.tril(np.ones((M, N), dtype=bool)), S, -np.inf)
    P = np.exp(S - L[:, None])
    dP = g @ v.T
    delta = (O * g).sum(-1)
    dabs = np.abs(O * g).sum(-1)
    dq_ref, dk_ref, dv_ref = refs
    sc = abs(scale)
    h = H_F16 if u == U_F16 else H_BF16

    def bound(w, x, n, ref, coherent=0.0, hs=1.0):
        # element (a, d) = sum_i w[i, a] * x[i, d] with w, x >= 0
        rss = np.sqrt((w * w).T @ (x * x))
        s1 = w.T @ x
        live = (w > 0).astype(np.float64)
        under = LAMBDA * h * hs * np.sqrt(live.T @ (x * x))
        return (LAMBDA * u * rss + LAMBDA * np.sqrt(n) * U_F32 * s1
                + u * np.abs(ref) + h * (ref != 0) + under + coherent)

    b_dv = bound(P, np.abs(g), M, dv_ref)
    wk = sc * P * (np.abs(dP) + np.abs(delta)[:, None] + dabs[:, None])
    b_dk = bound(wk, np.abs(q), M, dk_ref, hs=sc)
    wq = sc * P * (np.abs(dP) + np.abs(delta)[:, None])
    coh = 2.0 * u * sc * dabs[:, None] * (P @ np.abs(k))
    b_dq = bound(wq.T, np.abs(k), N, dq_ref, coherent=coh, hs=sc)
    return b_dq, b_dk, b_dv


def check_heads(q, k, v, g, causal, scale, heads=None, label="", one_pass=True):
    """GPU forward + backward on the full tensors; every element of the
    listed heads (default: all) against the oracle within head_bounds."""
    B, H, M, D = q.shape
    N = k.shape[2]
    print(f"[bwd-parity] {label} {tuple(q.shape)} N={N} causal={causal} scale={scale} "
          f"one_pass={one_pass}", flush=True)
    dq, dk, dv, _, _ = gpu_fwd_bwd(q, k, v, g, causal, scale, one_pass)
    for t in (dq, dk, dv):
        assert np.isfinite(t).all(), "non-finite gradient"
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    refs = oracle.attn_bwd_heads(q, k, v, g, heads, is_causal=causal, scale=scale)
    worst = {}
    for (b, h), ref in zip(heads, refs):
        f64 = lambda t: t[b, h].double().numpy()
        u = U_F16 if q.dtype == torch.float16 else U_BF16
        bounds = head_bounds(f64(q), f64(k), f64(v), f64(g), scale, causal, ref, u)
        for name, got, r, bd in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref, bounds):
            err = np.abs(got[b, h] - r)
            # a zero bound (every term zero, e.g. keys no query sees) needs
            # an exact zero
            with np.errstate(divide="ignore", invalid="ignore"):
                rel = np.where(bd > 0, err / bd, np.where(err > 0, np.inf, 0.0))
            ratio = float(rel.max(initial=0.0))
            worst[name] = max(worst.get(name, 0.0), ratio)
            assert ratio <= 1.0, (f"{label} head {(b, h)} {name}: max |err| / bound = "
                                  f"{ratio:.3g} (max |err| {err.max():.3g})")
    return worst
