"""Pins for the fp64 gradient oracle (oracle.attn_bwd), against things other
than itself.

* central finite differences of the forward oracle (itself pinned in
  test_oracle_pins.py): every element of dQ, dK and dV on tiny inputs, causal
  and not -- a dropped term, a wrong sign, a transposed operand or a missing
  scale fails here;
* torch's fp64 CPU autograd through scaled_dot_product_attention (a library
  routine);
* an fp64 numpy restatement of the tiled backward of "Blackwell Attention
  Example" (backward kernel implementation section): base-2 probabilities
  from the base-2 logsumexp and pre-scaled keys, the row term from
  rowsum(O * dO) (preprocess kernel), dQ scaled by ln 2 and dK by the softmax
  scale, over several tile sizes;
* closed forms and invariants: scale 0, one key, constant V, zero dO,
  keys' gradients summing to zero, the identity sum_i q_i.dQ_i = sum_j k_j.dK_j,
  linearity in dO, joint key permutation, the scale derivative.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from scaled_dot_product_12_amd.inputs import make_qkv, make_dout


def _rand(B, H, M, N, D, seed):
    q, k, v = make_qkv(B, H, M, N, D, "fp32", seed)
    g = make_dout(B, H, M, D, "fp32", seed)
    return tuple(t.double().numpy() for t in (q, k, v, g))


def _objective(q, k, v, g, causal, scale):
    """f = sum(O * dO): its gradient in (q, k, v) is what attn_bwd returns."""
    o, _ = oracle.attn_fwd(q, k, v, is_causal=causal, scale=scale, nthreads=1)
    return float((o * g).sum())


# --------------------------------------------------- finite differences
@pytest.mark.parametrize("M,N,D", [(3, 4, 2), (5, 3, 3), (4, 4, 2), (1, 3, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_central_differences(M, N, D, causal):
    q, k, v, g = _rand(1, 2, M, N, D, seed=40 + M * 7 + N)
    scale = 0.8
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=scale)
    h = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep = x[idx]
            x[idx] = keep + h
            fp = _objective(q, k, v, g, causal, scale)
            x[idx] = keep - h
            fm = _objective(q, k, v, g, causal, scale)
            x[idx] = keep
            fd[idx] = (fp - fm) / (2 * h)
        err = np.abs(grad - fd).max()
        assert err <= 1e-7, f"d{name}: max |analytic - central difference| = {err:.3g}"


def test_scale_derivative():
    """d f / d scale = sum_ij dS_ij <q_i, k_j> = sum_i <q_i, dQ_i> / scale."""
    q, k, v, g = _rand(1, 1, 6, 7, 4, seed=48)
    for causal in (False, True):
        scale, h = 0.6, 1e-6
        dq, _, _ = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=scale)
        fd = (_objective(q, k, v, g, causal, scale + h)
              - _objective(q, k, v, g, causal, scale - h)) / (2 * h)
        assert abs((q * dq).sum() / scale - fd) <= 1e-7


# ------------------------------------------------------ library routine
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N,D", [(33, 33, 16), (17, 40, 32), (40, 17, 8), (64, 64, 64)])
def test_torch_autograd(causal, M, N, D):
    q, k, v, g = _rand(2, 3, M, N, D, seed=50 + D)
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=scale)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                         scale=scale)
    o.backward(torch.from_numpy(g))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() <= 1e-12


# ------------------------------------- the pages' tiled backward in fp64
def _tiled_backward(q, k, v, g, o, lse, scale, block_m, block_n):
    """fp64 restatement of the tiled backward of "Blackwell Attention
    Example": keys pre-scaled by scale * log2(e), base-2 logsumexp, the row
    term delta = rowsum(O * dO) (preprocess kernel); for every key tile, a
    loop over query tiles accumulates dV and dK and adds each tile's dQ
    share (times ln 2); dK is multiplied by the softmax scale at the end.
    (The page writes ln 2 as the fp32 value 0.6931471824645996, whose product
    with the fp64 log2(e) it uses is 1 + 2.9e-9; the exact fp64 constants are
    used here so that the comparison can be made at 1e-12.) Non-causal, as on
    the page; tiles may be ragged."""
    log2e, ln2 = 1.0 / math.log(2.0), math.log(2.0)
    M, N = q.shape[0], k.shape[0]
    ks = k * (scale * log2e)
    lse2 = lse * log2e
    delta = (o * g).sum(-1)
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for n0 in range(0, N, block_n):
        kj, vj = ks[n0:n0 + block_n], v[n0:n0 + block_n]
        dv_acc = np.zeros(vj.shape)
        dk_acc = np.zeros(kj.shape)
        for m0 in range(0, M, block_m):
            qi, gi = q[m0:m0 + block_m], g[m0:m0 + block_m]
            p_t = np.exp2(kj @ qi.T - lse2[m0:m0 + block_m][None, :])
            dp_t = vj @ gi.T
            dv_acc += p_t @ gi
            ds_t = p_t * (dp_t - delta[m0:m0 + block_m][None, :])
            dq[m0:m0 + block_m] += (ds_t.T @ kj) * ln2
            dk_acc += ds_t @ qi
        dv[n0:n0 + block_n] = dv_acc
        dk[n0:n0 + block_n] = dk_acc * scale
    return dq, dk, dv


@pytest.mark.parametrize("block_m,block_n", [(64, 128), (16, 16), (7, 5), (1, 3)])
@pytest.mark.parametrize("M,N", [(32, 32), (29, 45)])
def test_pages_tiled_backward(block_m, block_n, M, N):
    q, k, v, g = _rand(1, 2, M, N, 16, seed=60 + M)
    scale = 0.25
    o, lse = oracle.attn_fwd(q, k, v, scale=scale)
    dq, dk, dv = oracle.attn_bwd(q, k, v, g, scale=scale)
    for h in range(2):
        tq, tk, tv = _tiled_backward(q[0, h], k[0, h], v[0, h], g[0, h], o[0, h],
                                     lse[0, h], scale, block_m, block_n)
        assert np.abs(dq[0, h] - tq).max() <= 1e-12
        assert np.abs(dk[0, h] - tk).max() <= 1e-12
        assert np.abs(dv[0, h] - tv).max() <= 1e-12


# -------------------------------------------------- closed forms / laws
def test_scale_zero():
    """Uniform probabilities over the visible keys: dQ = dK = 0 and
    dV_j = sum over the rows that see key j of dO_i / (number of keys row i sees)."""
    q, k, v, g = _rand(1, 2, 9, 6, 4, seed=70)
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=0.0)
        assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
        ref = np.zeros_like(dv)
        for i in range(9):
            n = min(i + 1, 6) if causal else 6
            ref[:, :, :n] += g[:, :, i:i + 1] / n
        assert np.abs(dv - ref).max() <= 1e-14


def test_single_key():
    q, k, v, g = _rand(2, 1, 5, 1, 8, seed=71)
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=0.3)
        assert np.abs(dq).max() == 0.0 and np.abs(dk).max() == 0.0
        assert np.abs(dv[:, :, 0] - g.sum(axis=2)).max() <= 1e-14


def test_constant_v_and_zero_dout():
    q, k, _, g = _rand(1, 2, 12, 10, 8, seed=72)
    v = np.full(k.shape, 0.75)
    for causal in (False, True):
        dq, dk, _ = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=0.5)
        assert np.abs(dq).max() <= 1e-14 and np.abs(dk).max() <= 1e-14
        z = oracle.attn_bwd(q, k, v, np.zeros_like(g), is_causal=causal, scale=0.5)
        assert all(np.abs(t).max() == 0.0 for t in z)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero_and_dot_identity(causal):
    """Adding one vector u to every key leaves O unchanged (each row's scores
    move by a constant), so sum_j dK_j = 0; and sum_i <q_i, dQ_i> equals
    sum_j <k_j, dK_j> (both are sum_ij dS_ij s_ij)."""
    q, k, v, g = _rand(2, 2, 16, 21, 8, seed=73)
    dq, dk, _ = oracle.attn_bwd(q, k, v, g, is_causal=causal, scale=0.45)
    assert np.abs(dk.sum(axis=2)).max() <= 1e-13
    lhs = (q * dq).sum(axis=(2, 3))
    rhs = (k * dk).sum(axis=(2, 3))
    assert np.abs(lhs - rhs).max() <= 1e-12


def test_linear_in_dout_and_key_permutation():
    q, k, v, g = _rand(1, 2, 11, 13, 8, seed=74)
    g2 = np.random.default_rng(1).standard_normal(g.shape)
    a = oracle.attn_bwd(q, k, v, 2.0 * g - 3.0 * g2, scale=0.5)
    b = oracle.attn_bwd(q, k, v, g, scale=0.5)
    c = oracle.attn_bwd(q, k, v, g2, scale=0.5)
    for x, y, z in zip(a, b, c):
        assert np.abs(x - (2.0 * y - 3.0 * z)).max() <= 1e-12
    pk = np.random.default_rng(2).permutation(13)
    dq, dk, dv = oracle.attn_bwd(q, k[:, :, pk], v[:, :, pk], g, scale=0.5)
    assert np.abs(dq - b[0]).max() <= 1e-13
    assert np.abs(dk - b[1][:, :, pk]).max() <= 1e-13
    assert np.abs(dv - b[2][:, :, pk]).max() <= 1e-13


def test_heads_api_threads_and_arguments():
    q, k, v, g = _rand(2, 3, 19, 23, 16, seed=75)
    full = oracle.attn_bwd(q, k, v, g, is_causal=True, scale=0.25, nthreads=1)
    again = oracle.attn_bwd(q, k, v, g, is_causal=True, scale=0.25, nthreads=7)
    assert all(np.array_equal(x, y) for x, y in zip(full, again))
    heads = [(1, 2), (0, 0)]
    for (b, h), got in zip(heads, oracle.attn_bwd_heads(q, k, v, g, heads,
                                                        is_causal=True, scale=0.25)):
        for x, y in zip(got, full):
            assert np.array_equal(x, y[b, h])
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, k, v, g[:, :, :5])
    with pytest.raises(ValueError):
        oracle.attn_bwd_heads(q, k, v, g, [(2, 0)])
