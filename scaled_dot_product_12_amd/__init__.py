"""Python binding of libmi355_attn (the C ABI in include/mi355_attn.h).

Argument marshalling only: every step of the attention forward runs in the
library's HIP kernels. torch provides device memory and the current stream.
The C entry points are exposed under their own names; ``attn_fwd`` here takes
torch tensors, allocates O and L, and calls the C ``attn_fwd`` on torch's
current stream -- the interface of the pages' wrappers
(``flash_attention_reference(Q, K, V, is_causal=False, scale=None) -> (O, L)``
in "Extend Thunder with CUDA-Python"; ``(q, k, v) -> (o, lse)`` in
"Blackwell Attention Example"). ``attn_bwd`` takes the forward's inputs and
outputs and the upstream gradient dO and returns (dQ, dK, dV), as the
backward of that page's autograd function does. ``axial_pass`` and
``axial_block`` run the fused axial-attention block (LayerNorm, QKV
projection, per-head attention, output projection, residual) of the
PopcornBench axial-attention trajectory on an fp32 image [B, Hh, W, C].

There is no fallback: if the HIP library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmi355_attn.so")

# Mirrors of the header's constants.
MI355_ATTN_FP32 = 0
MI355_ATTN_BF16 = 1
MI355_ATTN_FP16 = 2
MI355_ATTN_OK = 0
MI355_ATTN_ERR_INVALID_ARG = 1
MI355_ATTN_ERR_UNSUPPORTED = 2
MI355_ATTN_ERR_MISALIGNED = 3
MI355_ATTN_ERR_HIP = 4
MI355_ATTN_ERR_SCRATCH = 5
MI355_ATTN_NOALLOC_MAX_ROWS = 1048576
MI355_ATTN_PATH_AUTO = 0
MI355_ATTN_PATH_MAIN = 1
MI355_ATTN_PATH_SMALL = 2
MI355_AXIAL_ROW = 0
MI355_AXIAL_COL = 1

EXPORTS = ("attn_fwd", "attn_fwd_validate", "attn_fwd_path",
           "attn_fwd_select_path", "attn_status_string", "attn_bwd",
           "attn_bwd_validate", "axial_pass", "axial_pass_validate", "axial_block",
           "attn_fwd_dv", "attn_fwd_dv_validate", "axial_pass_split",
           "attn_bwd_noalloc", "attn_fwd_fp8", "attn_fwd_fp8_validate",
           "attn_bwd_ws", "attn_bwd_work_bytes", "attn_bwd_work_error_offset")

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, cint = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                               ctypes.c_float, cint, cint, vp]
        L.attn_fwd.restype = cint
        L.attn_fwd_path.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                    ctypes.c_float, cint, cint, cint, vp]
        L.attn_fwd_path.restype = cint
        L.attn_fwd_validate.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                        i64, ctypes.c_float, cint, cint]
        L.attn_fwd_validate.restype = cint
        L.attn_fwd_select_path.argtypes = [i64, i64, i64, i64, i64, cint, cint]
        L.attn_fwd_select_path.restype = cint
        L.attn_bwd.argtypes = [vp] * 10 + [i64] * 5 + [ctypes.c_float, cint, cint, vp]
        L.attn_bwd.restype = cint
        L.attn_bwd_noalloc.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_float, cint, cint, vp]
        L.attn_bwd_noalloc.restype = cint
        L.attn_bwd_ws.argtypes = ([vp] * 10 + [i64] * 5 + [ctypes.c_float, cint, cint, vp, i64,
                                                           vp])
        L.attn_bwd_ws.restype = cint
        L.attn_bwd_work_bytes.argtypes = [i64] * 5 + [cint, cint]
        L.attn_bwd_work_bytes.restype = i64
        L.attn_bwd_work_error_offset.argtypes = []
        L.attn_bwd_work_error_offset.restype = cint
        L.attn_fwd_fp8.argtypes = [vp] * 5 + [i64] * 5 + [ctypes.c_float, cint, vp]
        L.attn_fwd_fp8.restype = cint
        L.attn_fwd_fp8_validate.argtypes = [vp] * 5 + [i64] * 5 + [ctypes.c_float, cint]
        L.attn_fwd_fp8_validate.restype = cint
        L.attn_bwd_validate.argtypes = [vp] * 10 + [i64] * 5 + [ctypes.c_float, cint, cint]
        L.attn_bwd_validate.restype = cint
        L.attn_fwd_dv.argtypes = [vp] * 5 + [i64] * 6 + [ctypes.c_float, cint, cint, vp]
        L.attn_fwd_dv.restype = cint
        L.attn_fwd_dv_validate.argtypes = [vp] * 5 + [i64] * 6 + [ctypes.c_float, cint, cint]
        L.attn_fwd_dv_validate.restype = cint
        L.axial_pass.argtypes = [vp] * 7 + [i64] * 5 + [cint, ctypes.c_float, vp]
        L.axial_pass.restype = cint
        L.axial_pass_validate.argtypes = [vp] * 7 + [i64] * 5 + [cint, ctypes.c_float]
        L.axial_pass_validate.restype = cint
        L.axial_pass_split.argtypes = [vp, vp, i64, i64, i64, cint]
        L.axial_pass_split.restype = cint
        L.axial_block.argtypes = [vp] * 12 + [i64] * 5 + [ctypes.c_float, vp]
        L.axial_block.restype = cint
        L.attn_status_string.argtypes = [cint]
        L.attn_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


def attn_fwd_validate(q, k, v, o, lse, B, H, M, N, D, scale, is_causal, dtype) -> int:
    """Status attn_fwd would return; pointers are ints (addresses) or None."""
    return lib().attn_fwd_validate(q, k, v, o, lse, B, H, M, N, D, float(scale),
                                   int(is_causal), int(dtype))


def attn_bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N, D, scale,
                      is_causal, dtype) -> int:
    """Status attn_bwd would return; pointers are ints (addresses) or None."""
    return lib().attn_bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, M, N,
                                   D, float(scale), int(is_causal), int(dtype))


def attn_fwd_select_path(B, H, M, N, D, is_causal, dtype) -> int:
    return lib().attn_fwd_select_path(B, H, M, N, D, int(is_causal), int(dtype))


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to fp32, the value the C ABI receives by default."""
    return ctypes.c_float(1.0 / math.sqrt(D)).value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MI355_ATTN_FP32
    if t.dtype == torch.bfloat16:
        return MI355_ATTN_BF16
    if t.dtype == torch.float16:
        return MI355_ATTN_FP16
    raise ValueError(f"unsupported dtype {t.dtype}: use float32, bfloat16 or float16")


def _check(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, seq, D]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share one dtype")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, M, D = q.shape
    if (k.shape[0] != B or k.shape[1] != H or k.shape[3] != D
            or v.shape[:3] != k.shape[:3]):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"v {tuple(v.shape)}")
    return B, H, M, k.shape[2], D


def attn_fwd(q, k, v, is_causal: bool = False, scale: Optional[float] = None,
             out: Optional[Tuple] = None,
             path: int = MI355_ATTN_PATH_AUTO):
    """(O, L) = attention forward of GPU tensors q [B,H,M,D], k [B,H,N,D],
    v [B,H,N,Dv] (Dv = D, or through the C attn_fwd_dv any other of 16, 32,
    64, 128: O is then [B,H,M,Dv]).

    O has q's dtype; L is fp32 [B,H,M], natural log. ``scale`` defaults to
    1/sqrt(D). ``out=(o, lse)`` writes into preallocated tensors. ``path``
    forces a kernel (MI355_ATTN_PATH_MAIN / _SMALL); the default lets the
    library choose. The call is asynchronous on torch's current stream.
    """
    import torch
    B, H, M, N, D = _check(q, k, v)
    Dv = v.shape[3]
    dt = _dtype_code(q)
    if scale is None:
        scale = default_scale(D)
    if Dv != D and path != MI355_ATTN_PATH_AUTO:
        raise ValueError("a value head dim other than D takes the default path")
    if out is None:
        o = q.new_empty((B, H, M, Dv))
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if (tuple(o.shape) != (B, H, M, Dv) or o.dtype != q.dtype
                or not o.is_contiguous()):
            raise ValueError("out[0] must be a contiguous [B, H, M, Dv] tensor of q's dtype")
        if (tuple(lse.shape) != (B, H, M) or lse.dtype != torch.float32
                or not lse.is_contiguous()):
            raise ValueError("out[1] must be a contiguous fp32 [B, H, M] tensor")
        if o.device != q.device or lse.device != q.device:
            raise ValueError("out tensors must be on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if Dv != D:
            st = lib().attn_fwd_dv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), B, H, M, N, D, Dv, float(scale),
                                   int(bool(is_causal)), dt, stream)
        else:
            st = lib().attn_fwd_path(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     o.data_ptr(), lse.data_ptr(), B, H, M, N, D,
                                     float(scale), int(bool(is_causal)), dt,
                                     int(path), stream)
    if st != MI355_ATTN_OK:
        raise RuntimeError(f"attn_fwd failed: {attn_status_string(st)} ({st})")
    return o, lse


def attn_fwd_fp8_validate(q, k, vt, o, lse, B, H, M, N, D, scale, is_causal) -> int:
    """Status attn_fwd_fp8 would return; pointers are ints (addresses) or None."""
    return lib().attn_fwd_fp8_validate(q, k, vt, o, lse, B, H, M, N, D, float(scale),
                                       int(is_causal))


def attn_fwd_fp8(q, k, vt, is_causal: bool = False, scale: Optional[float] = None,
                 out: Optional[Tuple] = None):
    """(O, L) of attention on fp8 inputs: q [B,H,M,D] and k [B,H,N,D] as
    torch.float8_e4m3fn, vt = V transposed, [B,H,D,N] float8_e4m3fn (as the
    Blackwell example takes fp8 values). O is bf16 [B,H,M,D], L fp32 [B,H,M].
    D in {64, 128}, N a multiple of 16. Asynchronous on torch's current stream.
    """
    import torch
    f8 = torch.float8_e4m3fn
    for name, t in (("q", q), ("k", k), ("vt", vt)):
        if t.device.type != "cuda" or t.dtype != f8 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-D float8_e4m3fn GPU tensor")
    if not (q.device == k.device == vt.device):
        raise ValueError("q, k, vt must be on one device")
    B, H, M, D = q.shape
    N = k.shape[2]
    if tuple(k.shape) != (B, H, N, D) or tuple(vt.shape) != (B, H, D, N):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"vt {tuple(vt.shape)} (vt is [B, H, D, N])")
    if scale is None:
        scale = default_scale(D)
    if out is None:
        o = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        if (tuple(o.shape) != (B, H, M, D) or o.dtype != torch.bfloat16
                or not o.is_contiguous() or o.device != q.device):
            raise ValueError("out[0] must be a contiguous bf16 [B, H, M, D] tensor on q's device")
        if (tuple(lse.shape) != (B, H, M) or lse.dtype != torch.float32
                or not lse.is_contiguous() or lse.device != q.device):
            raise ValueError("out[1] must be a contiguous fp32 [B, H, M] tensor on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = lib().attn_fwd_fp8(q.data_ptr(), k.data_ptr(), vt.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), B, H, M, N, D, float(scale),
                                int(bool(is_causal)), stream)
    if st != MI355_ATTN_OK:
        raise RuntimeError(f"attn_fwd_fp8 failed: {attn_status_string(st)} ({st})")
    return o, lse


def attn_bwd_work_bytes(B, H, M, N, D, is_causal, dtype) -> int:
    """Work-area bytes for the one-pass backward (0 where it does not apply)."""
    return lib().attn_bwd_work_bytes(B, H, M, N, D, int(bool(is_causal)), int(dtype))


def attn_bwd_work_error_offset() -> int:
    return lib().attn_bwd_work_error_offset()


def attn_bwd(q, k, v, o, lse, dout, is_causal: bool = False,
             scale: Optional[float] = None, out: Optional[Tuple] = None,
             delta=None, one_pass: bool = True, work=None):
    """(dQ, dK, dV) of attention for the upstream gradient ``dout``.

    ``q, k, v`` are the forward's inputs, ``o, lse`` its outputs (from
    ``attn_fwd`` with the same ``is_causal`` and ``scale``), ``dout`` has o's
    shape and dtype. Gradients have the inputs' dtype. ``out=(dq, dk, dv)``
    writes into preallocated tensors; ``delta`` is an optional fp32 [B, H, M]
    workspace (allocated here if None) that receives rowsum(O * dO). bf16
    or fp16, D in {32, 64, 128}. Asynchronous on torch's current stream.

    Where the one-pass backward applies (D = 128, no mask) and ``one_pass``
    is true, the call goes through the C ``attn_bwd_ws``
    with a work area (``work``: a uint8 GPU tensor of at least
    ``attn_bwd_work_bytes`` bytes, allocated here if None); otherwise through
    ``attn_bwd``. Both are deterministic.
    """
    import torch
    B, H, M, N, D = _check(q, k, v)
    if v.shape != k.shape:
        raise ValueError("attn_bwd needs v with the head dim of q and k")
    dt = _dtype_code(q)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape)):
        if (t.shape != shape or t.dtype != q.dtype or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if (tuple(lse.shape) != (B, H, M) or lse.dtype != torch.float32
            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 [B, H, M] tensor on q's device")
    if scale is None:
        scale = default_scale(D)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    else:
        dq, dk, dv = out
        for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
            if (t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous()
                    or t.device != q.device):
                raise ValueError(f"out {name} must be a contiguous tensor like {name[1]}")
    if delta is None:
        delta = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    elif (tuple(delta.shape) != (B, H, M) or delta.dtype != torch.float32
          or not delta.is_contiguous() or delta.device != q.device):
        raise ValueError("delta must be a contiguous fp32 [B, H, M] tensor on q's device")
    need = attn_bwd_work_bytes(B, H, M, N, D, is_causal, dt) if one_pass else 0
    if need > 0:
        if work is None:
            work = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif (work.dtype != torch.uint8 or work.device != q.device or not work.is_contiguous()
              or work.numel() < need):
            raise ValueError(f"work must be a contiguous uint8 tensor of >= {need} bytes "
                             "on q's device")
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if need > 0:
            st = lib().attn_bwd_ws(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, M, N,
                                   D, float(scale), int(bool(is_causal)), dt, work.data_ptr(),
                                   work.numel(), stream)
        else:
            st = lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), delta.data_ptr(), B, H, M, N, D, float(scale),
                                int(bool(is_causal)), dt, stream)
    if st != MI355_ATTN_OK:
        name = "attn_bwd_ws" if need > 0 else "attn_bwd"
        raise RuntimeError(f"{name} failed: {attn_status_string(st)} ({st})")
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, dout, out, is_causal: bool = False,
                     scale: Optional[float] = None):
    """attn_bwd through the C ``attn_bwd_noalloc``: no workspace argument and
    no allocation on this path -- the caller passes ``out=(dq, dk, dv)``
    (contiguous tensors like q, k, v) and the library keeps delta in its
    static device array (B*H*M <= MI355_ATTN_NOALLOC_MAX_ROWS). Calls that
    overlap on one GPU share that array and must not run concurrently."""
    import torch
    B, H, M, N, D = _check(q, k, v)
    if v.shape != k.shape:
        raise ValueError("attn_bwd_noalloc needs v with the head dim of q and k")
    dt = _dtype_code(q)
    for name, t, shape in (("o", o, q.shape), ("dout", dout, q.shape)):
        if (t.shape != shape or t.dtype != q.dtype or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError(f"{name} must be a contiguous tensor like q")
    if (tuple(lse.shape) != (B, H, M) or lse.dtype != torch.float32
            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 [B, H, M] tensor on q's device")
    dq, dk, dv = out
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if (t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError(f"out {name} must be a contiguous tensor like {name[1]}")
    if scale is None:
        scale = default_scale(D)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        st = lib().attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                    dk.data_ptr(), dv.data_ptr(), B, H, M, N, D,
                                    float(scale), int(bool(is_causal)), dt, stream)
    if st != MI355_ATTN_OK:
        raise RuntimeError(f"attn_bwd_noalloc failed: {attn_status_string(st)} ({st})")
    return dq, dk, dv


def axial_pass_validate(x, out, ln_w, ln_b, w_qkv, w_out, b_out, B, Hh, W, C, heads,
                        axis, eps) -> int:
    """The C checks of axial_pass on raw pointers (integers); no launch."""
    return lib().axial_pass_validate(x, out, ln_w, ln_b, w_qkv, w_out, b_out, B, Hh, W, C,
                                     heads, int(axis), float(eps))


def axial_pass_split(x, out, B, Hh, W, axis) -> int:
    """Workgroups per sequence of axial_pass's launch (2 or 1; -1 if invalid);
    x and out are addresses (integers). Host logic only."""
    return lib().axial_pass_split(x, out, B, Hh, W, int(axis))


def _check_axial(x, params, out):
    import torch
    if x.device.type != "cuda" or x.dtype != torch.float32 or x.dim() != 4:
        raise ValueError("x must be an fp32 GPU tensor [B, Hh, W, C]")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    C = x.shape[3]
    want = ((C,), (C,), (3 * C, C), (C, C), (C,))
    if len(params) != 5:
        raise ValueError("params are (ln_w, ln_b, w_qkv, w_out, b_out)")
    for t, shp in zip(params, want):
        if (t.device != x.device or t.dtype != torch.float32 or tuple(t.shape) != shp
                or not t.is_contiguous()):
            raise ValueError(f"weights must be contiguous fp32 tensors of shapes {want} "
                             "on x's device")
    if out is None:
        out = torch.empty_like(x)
    elif (out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous()
          or out.device != x.device):
        raise ValueError("out must be a contiguous tensor like x")
    return out


def axial_pass(x, params, axis: int, heads: int = 4, eps: float = 1e-5, out=None):
    """One residual axial-attention pass of the fp32 image x [B, Hh, W, C].

    ``params`` = (ln_w [C], ln_b [C], w_qkv [3C, C], w_out [C, C], b_out [C]);
    ``axis`` MI355_AXIAL_ROW (sequences along W) or MI355_AXIAL_COL (along Hh).
    ``out`` may be x itself. Asynchronous on torch's current stream.
    """
    import torch
    out = _check_axial(x, params, out)
    B, Hh, W, C = x.shape
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = lib().axial_pass(x.data_ptr(), out.data_ptr(), *(t.data_ptr() for t in params),
                              B, Hh, W, C, int(heads), int(axis), float(eps), stream)
    if st != MI355_ATTN_OK:
        raise RuntimeError(f"axial_pass failed: {attn_status_string(st)} ({st})")
    return out


def axial_block(x, row_params, col_params, heads: int = 4, eps: float = 1e-5, out=None):
    """The row pass into ``out``, then the column pass on ``out`` in place."""
    import torch
    out = _check_axial(x, row_params, out)
    _check_axial(x, col_params, out)
    B, Hh, W, C = x.shape
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = lib().axial_block(x.data_ptr(), out.data_ptr(),
                               *(t.data_ptr() for t in row_params),
                               *(t.data_ptr() for t in col_params),
                               B, Hh, W, C, int(heads), float(eps), stream)
    if st != MI355_ATTN_OK:
        raise RuntimeError(f"axial_block failed: {attn_status_string(st)} ({st})")
    return out
