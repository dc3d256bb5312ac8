"""fp64 CPU oracle for the fused axial-attention block (row pass, then column pass).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP path and imports nothing from it.

Source: the PopcornBench axial-attention trajectory (the model's reference
forward and its per-pass attention helper). An image tensor x [B, Hh, W, C]
goes through two residual attention passes:

* row pass: each image row (b, y) is a sequence of W tokens;
* column pass, on the row pass's output: each image column (b, x) is a
  sequence of Hh tokens.

One pass, for every sequence of tokens t (feature vectors of length C):
  1. LayerNorm over the C features, biased variance, eps added to it, then the
     affine weight and bias;
  2. a bias-free linear layer to 3C features, read as (Q, K, V) each split into
     ``heads`` heads of C / heads features (the view [L, 3, heads, d]);
  3. per head, softmax(Q K^T / sqrt(d)) V over the sequence (no mask);
  4. heads concatenated back to C features, then a linear layer with bias;
  5. the result added to the pass's input at the same (b, y, x) position.

Linear layers follow torch's convention y = x W^T (+ b) with W stored
[out_features, in_features]. Everything is evaluated in IEEE fp64 with numpy
(matrix products by ``@``); inputs are widened exactly.

Parity pins (tests/test_oracle_axial_pins.py): torch's fp64 modules built from
the same description, closed forms (zero output projection, zero key
projection, one-token sequences), the row/column transpose relation and token
permutation equivariance.
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np


class PassParams(NamedTuple):
    """Weights of one pass: LayerNorm (ln_w, ln_b) [C], QKV [3C, C], out [C, C], out bias [C]."""
    ln_w: np.ndarray
    ln_b: np.ndarray
    w_qkv: np.ndarray
    w_out: np.ndarray
    b_out: np.ndarray


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float64).contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def params_f64(p) -> PassParams:
    return PassParams(*(_f64(t) for t in p))


def layer_norm(x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    """Step 1 over the last axis: (x - mean) / sqrt(var + eps) * w + b, var biased."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * w + b


def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Step 3 for arrays [..., L, d]: softmax over keys of q k^T / sqrt(d), times v."""
    d = q.shape[-1]
    s = q @ np.swapaxes(k, -1, -2) / np.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return (e / e.sum(axis=-1, keepdims=True)) @ v


def attend_sequences(seqs: np.ndarray, p: PassParams, heads: int, eps: float) -> np.ndarray:
    """Steps 1-4 for seqs [S, L, C]; returns the pass's update [S, L, C] (no residual)."""
    S, L, C = seqs.shape
    d = C // heads
    xn = layer_norm(seqs, p.ln_w, p.ln_b, eps)
    qkv = (xn @ p.w_qkv.T).reshape(S, L, 3, heads, d)
    q, k, v = (np.transpose(qkv[:, :, i], (0, 2, 1, 3)) for i in range(3))  # [S, h, L, d]
    o = softmax_attention(q, k, v)
    o = np.transpose(o, (0, 2, 1, 3)).reshape(S, L, C)
    return o @ p.w_out.T + p.b_out


def axial_pass(x, p, axis: str, heads: int, eps: float = 1e-5) -> np.ndarray:
    """One residual pass over x [B, Hh, W, C]; axis "row" (sequences along W) or "col"."""
    x = _f64(x)
    p = params_f64(p)
    B, Hh, W, C = x.shape
    if C % heads:
        raise ValueError("C must be a multiple of heads")
    if axis == "row":
        upd = attend_sequences(x.reshape(B * Hh, W, C), p, heads, eps).reshape(B, Hh, W, C)
    elif axis == "col":
        seqs = np.transpose(x, (0, 2, 1, 3)).reshape(B * W, Hh, C)
        upd = np.transpose(attend_sequences(seqs, p, heads, eps).reshape(B, W, Hh, C), (0, 2, 1, 3))
    else:
        raise ValueError("axis must be 'row' or 'col'")
    return x + upd


def axial_block(x, row_params, col_params, heads: int, eps: float = 1e-5) -> np.ndarray:
    """The row pass, then the column pass on its output (step 5 after each)."""
    return axial_pass(axial_pass(x, row_params, "row", heads, eps), col_params, "col", heads, eps)
