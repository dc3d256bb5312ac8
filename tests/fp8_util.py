"""The error bound of the fp8 forward (attn_fwd_fp8) against the fp64 oracle
run on the same e4m3 inputs, and helpers for its GPU parity tests.

What the kernel rounds (everything else is exact or fp32):
* the scores q.k of e4m3 inputs are exact products summed in fp32;
* P is rounded to e4m3 (round to nearest even) before the second product:
  relative error at most u = 2^-4 (4 significant bits) in the normal range,
  absolute error at most 2^-10 (half the smallest subnormal 2^-9) below it.
  The kernel's P is exp2 of the score minus a reference at most 8 (log2
  units) below the row max, so it is the oracle's P (max 1) times 2^a with
  0 <= a <= 8: the relative bound holds as is and the absolute one only
  shrinks when brought to the oracle's scale;
* the row sum is the fp32 sum of the same rounded P (so O is a convex
  combination of value rows), and O is rounded to bf16 on the store
  (u_bf16 = 2^-8).

With e_j = max(u P_j, 2^-10) the bound on the rounding error r_j of P_j
and l = sum_j P_j, exactly
    O_i - O_ref,i = sum_j r_j (v_j - O_ref,i) / (l + sum_j r_j),
where the r_j are independent with |r_j| <= e_j; by Hoeffding's inequality
the numerator stays below lambda * sqrt(sum_j e_j^2 (v_j - O_i)^2) except
with probability 2 exp(-lambda^2 / 2) ~ 2.5e-14 per element (lambda = 8),
and the denominator is at least l - sum_j e_j. Likewise
L_i - L_ref,i = ln(1 + sum_j r_j / l), at most -ln(1 - t) with
t = lambda sqrt(sum_j e_j^2) / l. fp32 accumulation adds
lambda sqrt(n) 2^-24 sum_j w_j |v_jd| to O and a few 2^-24 |L| to L; the
fp32 sum of the D products of a score errs by at most
dx_j = D 2^-24 |scale| sum_d |q_d k_jd|, which moves L by at most max_j dx_j
and P_j by a factor within exp(+-dx_j), i.e. O by at most
2 max_j dx_j sum_j w_j |v_jd - O_d|.
"""
import numpy as np

import oracle

U_E4M3 = 2.0 ** -4
E4M3_SUB = 2.0 ** -10
U_BF16 = 2.0 ** -8
U_F32 = 2.0 ** -24
LAMBDA = 8.0


def head_bounds(q, k, v, scale, causal):
    """Per-element bounds (b_O [M, D], b_L [M]) and the oracle's (O, L) for
    one head of fp64 arrays q [M, D], k [N, D], v [N, D] (the e4m3 values)."""
    M, N = q.shape[0], k.shape[0]
    S = scale * (q @ k.T)
    if causal:
        S = np.where(np.arange(N)[None, :] <= np.arange(M)[:, None], S, -np.inf)
    m = S.max(1, keepdims=True)
    P = np.exp(S - m)
    l = P.sum(1, keepdims=True)
    O = (P @ v) / l
    L = (m + np.log(l))[:, 0]
    e = np.where(P > 0, np.maximum(U_E4M3 * P, E4M3_SUB), 0.0)
    E2 = (e / l) ** 2
    rss2 = E2 @ (v * v) - 2.0 * O * (E2 @ v) + O * O * E2.sum(1, keepdims=True)
    rss = np.sqrt(np.maximum(rss2, 0.0))
    shrink = np.maximum(1.0 - e.sum(1, keepdims=True) / l, 0.5)  # (l - sum e) / l
    n = max(N, 1)
    b_o = (LAMBDA * rss / shrink + U_BF16 * np.abs(O)
           + LAMBDA * np.sqrt(n) * U_F32 * ((P / l) @ np.abs(v)) + 4 * U_F32)
    D = q.shape[1]
    dx = D * U_F32 * abs(scale) * (np.abs(q) @ np.abs(k).T)
    dx_max = np.where(P > 0, dx, 0.0).max(1, keepdims=True)
    W = P / l
    spread = W @ np.abs(v) + np.abs(O)  # >= sum_j w_j |v_jd - O_d|
    b_o = b_o + 2.0 * dx_max * spread
    t = np.minimum(LAMBDA * np.sqrt(E2.sum(1)), 0.5)
    b_l = -np.log1p(-t) + 8 * U_F32 * (np.abs(L) + np.log(n) + 1.0) + dx_max[:, 0]
    return b_o, b_l, O, L


def check_fp8(q, k, v, causal, scale, o, lse, heads=None, label=""):
    """Every element of the listed heads (default: all) of the GPU outputs
    (o [B,H,M,D], lse [B,H,M] as numpy) within head_bounds of the oracle, which
    runs on the same e4m3 values (widened exactly). Returns the worst
    |err| / bound for O and L."""
    B, H = q.shape[:2]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{label}: non-finite output"
    worst_o = worst_l = 0.0
    f64 = lambda t, b, h: oracle._f64(t[b, h])
    for b, h in heads:
        bo, bl, _, _ = head_bounds(f64(q, b, h), f64(k, b, h), f64(v, b, h), scale, causal)
        sl = lambda t: t[b:b + 1, h:h + 1]
        ro, rl = oracle.attn_fwd(sl(q), sl(k), sl(v), is_causal=causal, scale=scale)
        ro, rl = ro[0, 0], rl[0, 0]
        eo = np.abs(o[b, h] - ro)
        el = np.abs(lse[b, h] - rl)
        ro_ = float((eo / bo).max(initial=0.0))
        rl_ = float((el / bl).max(initial=0.0))
        worst_o, worst_l = max(worst_o, ro_), max(worst_l, rl_)
        assert ro_ <= 1.0 and rl_ <= 1.0, (
            f"{label} head {(b, h)}: max |dO|/bound = {ro_:.3g} (max |dO| {eo.max():.3g}), "
            f"max |dL|/bound = {rl_:.3g} (max |dL| {el.max():.3g})")
    return worst_o, worst_l


def transpose_v(v):
    """[B, H, N, D] -> [B, H, D, N] contiguous (the fp8 kernel's value layout)."""
    return v.transpose(-1, -2).contiguous()
