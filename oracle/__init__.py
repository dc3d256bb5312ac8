"""fp64 CPU oracle for scaled-dot-product attention (O and the per-row logsumexp L).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP path (``scaled_dot_product_12_amd``) and neither imports the
other; both are fed by the seeded generators in
``scaled_dot_product_12_amd.inputs``, which hold none of the method's
arithmetic.

What it computes is the plain definition, row by row, in IEEE fp64 (see
``attn_oracle.c``): softmax(scale * Q K^T [+ top-left causal mask]) V and
L = max + ln(sum exp(s - max)). Sources: "Extend Thunder with CUDA-Python",
Python reference section (flash_attention_reference, whose tiled loop reduces
to this when one tile spans all keys, and whose causal mask keeps key <= query
in absolute positions); "Blackwell Attention Example", attention kernel (lse as
one value per query row, [B, H, M]).

Inputs are widened to fp64 exactly (fp32, bf16 and fp16 values are
representable), so for 16-bit inputs the oracle sees the rounded values the
GPU sees.

The gradient (``attn_bwd``, ``attn_bwd_heads``; see ``attn_oracle_bwd.c``) is
the chain rule through softmax attention, dQ, dK, dV for an upstream dO, with
the softmax Jacobian written out; "Blackwell Attention Example" (backward
kernel and autograd function sections) evaluates the same quantity tile by
tile.

Parity pins (tests/test_oracle_pins.py, tests/test_oracle_bwd_pins.py): a
50-digit ``decimal`` brute force, an independent fp64 re-implementation of the
pages' tiled online algorithm, torch's fp64 CPU SDPA, and closed forms /
invariants for the forward; central finite differences of the forward,
torch's fp64 autograd, an fp64 restatement of the pages' tiled backward, and
closed forms / invariants for the gradient. Every function here is pinned.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Iterable, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_attn.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_attn_fwd.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                        i64, ctypes.c_double, ctypes.c_int,
                                        ctypes.c_int]
        lib.oracle_attn_fwd.restype = ctypes.c_int
        lib.oracle_attn_rows.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, i64,
                                         i64, ctypes.c_double, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int64), i64,
                                         ctypes.c_int]
        lib.oracle_attn_rows.restype = ctypes.c_int
        lib.oracle_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, i64, i64, i64,
                                        i64, i64, ctypes.c_double, ctypes.c_int,
                                        ctypes.c_int]
        lib.oracle_attn_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def host_threads() -> int:
    """Threads the oracle uses by default: every core this process may run on."""
    return len(os.sched_getaffinity(0))


def _f64(x) -> np.ndarray:
    """Exact widening of an fp32 / bf16 / fp16 / fp64 array (numpy or torch) to fp64."""
    if hasattr(x, "detach"):  # torch tensor, possibly bf16 which numpy lacks
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float64).contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_scale(D: int) -> float:
    """1/sqrt(D), the scale the pages use when none is given (fp64)."""
    return 1.0 / math.sqrt(D)


def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("oracle expects [B,H,M,D] / [B,H,N,D] arrays")
    B, H, M, D = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    return B, H, M, k.shape[2], D


def attn_fwd(q, k, v, is_causal: bool = False, scale: float | None = None,
             nthreads: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Every row: returns (O [B,H,M,D], L [B,H,M]) as fp64 numpy arrays."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, M, N, D = _shapes(q, k, v)
    if scale is None:
        scale = default_scale(D)
    o = np.empty((B, H, M, D), dtype=np.float64)
    lse = np.empty((B, H, M), dtype=np.float64)
    rc = _load().oracle_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 B, H, M, N, D, float(scale), int(bool(is_causal)),
                                 nthreads or host_threads())
    if rc != 0:
        raise ValueError(f"oracle_attn_fwd failed with {rc}")
    return o, lse


def attn_rows(q, k, v, rows: Iterable[Tuple[int, int, int]],
              is_causal: bool = False, scale: float | None = None,
              nthreads: int | None = None) -> Tuple[np.ndarray, np.ndarray]:
    """Selected query rows (b, h, i): returns (O [n, D], L [n]) in fp64.

    Only the heads that the rows touch are widened, so this stays cheap on
    inputs far larger than the full oracle could finish.
    """
    rows = [tuple(int(t) for t in r) for r in rows]
    if q.ndim != 4:
        raise ValueError("oracle expects [B,H,M,D] arrays")
    B, H, M, D = q.shape
    N = k.shape[2]
    if scale is None:
        scale = default_scale(D)
    out_o = np.empty((len(rows), D), dtype=np.float64)
    out_l = np.empty((len(rows),), dtype=np.float64)
    by_head = {}
    for t, (b, h, i) in enumerate(rows):
        if not (0 <= b < B and 0 <= h < H and 0 <= i < M):
            raise ValueError(f"row {(b, h, i)} out of range")
        by_head.setdefault((b, h), []).append((t, i))
    lib = _load()
    for (b, h), items in by_head.items():
        qh, kh, vh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h])
        if kh.shape != (N, D) or vh.shape != (N, D):
            raise ValueError("k / v head shape mismatch")
        ids = np.array([i for _, i in items], dtype=np.int64)
        o = np.empty((len(items), D), dtype=np.float64)
        lse = np.empty((len(items),), dtype=np.float64)
        rc = lib.oracle_attn_rows(_ptr(qh), _ptr(kh), _ptr(vh), _ptr(o), _ptr(lse),
                                  1, 1, M, N, D, float(scale), int(bool(is_causal)),
                                  ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                  len(items), nthreads or host_threads())
        if rc != 0:
            raise ValueError(f"oracle_attn_rows failed with {rc}")
        for n, (t, _) in enumerate(items):
            out_o[t] = o[n]
            out_l[t] = lse[n]
    return out_o, out_l


def attn_bwd(q, k, v, dout, is_causal: bool = False, scale: float | None = None,
             nthreads: int | None = None):
    """Gradient of attention for upstream ``dout`` [B,H,M,D]: returns
    (dQ [B,H,M,D], dK [B,H,N,D], dV [B,H,N,D]) as fp64 numpy arrays."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, M, N, D = _shapes(q, k, v)
    if g.shape != q.shape:
        raise ValueError(f"dout {g.shape} must have q's shape {q.shape}")
    if M > 0 and N < 1:
        raise ValueError("no keys")
    if scale is None:
        scale = default_scale(D)
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(k.shape, dtype=np.float64)
    dv = np.empty(v.shape, dtype=np.float64)
    rc = _load().oracle_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(dq),
                                 _ptr(dk), _ptr(dv), B, H, M, N, D, float(scale),
                                 int(bool(is_causal)), nthreads or host_threads())
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd failed with {rc}")
    return dq, dk, dv


def attn_bwd_heads(q, k, v, dout, heads: Iterable[Tuple[int, int]],
                   is_causal: bool = False, scale: float | None = None,
                   nthreads: int | None = None):
    """Gradient for selected heads (b, h) only: returns lists of per-head
    (dQ [M,D], dK [N,D], dV [N,D]) in fp64, in the order given. Only those
    heads are widened, so this stays usable on inputs far larger than the
    full oracle could finish."""
    out = []
    for b, h in heads:
        b, h = int(b), int(h)
        if not (0 <= b < q.shape[0] and 0 <= h < q.shape[1]):
            raise ValueError(f"head {(b, h)} out of range")
        one = [x[b:b + 1, h:h + 1] for x in (q, k, v, dout)]
        dq, dk, dv = attn_bwd(*one, is_causal=is_causal, scale=scale,
                              nthreads=nthreads)
        out.append((dq[0, 0], dk[0, 0], dv[0, 0]))
    return out


def attn_fwd_dv(q, k, v, is_causal: bool = False, scale: float | None = None):
    """Attention whose values have their own head dim Dv (q, k [B,H,*,D],
    v [B,H,N,Dv]), as the Blackwell example's kernel allows: O [B,H,M,Dv] and
    L [B,H,M] in fp64. The plain definition with numpy products: scores
    scale * Q K^T (causal: key j <= query i), row max m, e = exp(s - m),
    O = e V / sum e, L = m + ln(sum e)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("oracle expects [B,H,M,D] / [B,H,N,D] / [B,H,N,Dv] arrays")
    B, H, M, D = q.shape
    N = k.shape[2]
    if k.shape != (B, H, N, D) or v.shape[:3] != (B, H, N):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if scale is None:
        scale = default_scale(D)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if is_causal:
        s = np.where(np.arange(N)[None, :] > np.arange(M)[:, None], -np.inf, s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return (e @ v) / l, (m + np.log(l))[..., 0]
