"""PyTorch-facing entry points over the library's C ABI: a differentiable
attention op and a drop-in for ``torch.nn.functional.scaled_dot_product_attention``.

* ``attention(q, k, v, is_causal, scale)`` is a ``torch.autograd.Function``
  whose forward is ``attn_fwd`` (saving q, k, v, O and L) and whose backward
  is ``attn_bwd`` -- the shape of the autograd function in "Blackwell
  Attention Example" (autograd function section).
* ``sdpa_checker`` takes torch's SDPA arguments and says whether this library
  implements that call, with the reason when it does not -- the checker of
  "Extend Thunder with CUDA-Python" (registering the kernel as an
  implementation of torch SDPA), extended to what the kernels here support
  (the causal mask; fp32, bf16 and fp16 forward; bf16 and fp16 backward).
* ``scaled_dot_product_attention`` has torch's signature; it runs the
  library's kernels when the checker accepts and raises NotImplementedError
  with the checker's reason otherwise. There is no silent fallback to another
  implementation.
* ``route_sdpa()`` is a context manager (a ``TorchFunctionMode``) under
  which every call of ``torch.nn.functional.scaled_dot_product_attention``
  made by unmodified user code -- a model's attention layer -- is offered to
  the checker and, when accepted, runs on the library's kernels: the
  executor / checker / implementation registration that "Extend Thunder with
  CUDA-Python" ("Running our kernel in Thunder") performs for its own
  kernel. A call the checker rejects raises NotImplementedError with the
  reason (``strict=True``, the default), or, with ``strict=False``, goes on
  to torch's own SDPA, as Thunder hands an operation its checker declines to
  the next executor in the list.

Inputs that are not contiguous are copied to contiguous [B, H, seq, D]
tensors first (a layout copy by torch; every step of the attention itself
runs in the library's kernels).
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import torch
from torch.overrides import TorchFunctionMode

from . import attn_bwd, attn_fwd

FWD_HEAD_DIMS = (16, 32, 64, 128)
BWD_HEAD_DIMS = (32, 64, 128)
BWD_DTYPES = (torch.bfloat16, torch.float16)


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, is_causal: bool, scale: Optional[float]):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = attn_fwd(q, k, v, is_causal=is_causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.is_causal, ctx.scale = is_causal, scale
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        if q.dtype not in BWD_DTYPES or q.shape[-1] not in BWD_HEAD_DIMS:
            raise NotImplementedError(
                f"attention backward supports bf16 and fp16 with head dim in {BWD_HEAD_DIMS}; "
                f"got {q.dtype}, D={q.shape[-1]}")
        dq, dk, dv = attn_bwd(q, k, v, o, lse, do.contiguous(), is_causal=ctx.is_causal,
                              scale=ctx.scale)
        return dq, dk, dv, None, None


def attention_with_lse(q, k, v, is_causal: bool = False,
                       scale: Optional[float] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """(O, L) like ``attn_fwd``, differentiable in q, k, v through O."""
    return _Attention.apply(q, k, v, bool(is_causal), scale)


def attention(q, k, v, is_causal: bool = False, scale: Optional[float] = None) -> torch.Tensor:
    """O = softmax(scale q k^T [+ causal mask]) v for [B, H, seq, D] GPU
    tensors, differentiable in q, k, v (backward: bf16 or fp16, D in 32/64/128)."""
    return _Attention.apply(q, k, v, bool(is_causal), scale)[0]


def sdpa_checker(query, key, value, attn_mask=None, dropout_p: float = 0.0,
                 is_causal: bool = False, scale: Optional[float] = None,
                 enable_gqa: bool = False) -> Tuple[bool, str]:
    """(True, "") when ``scaled_dot_product_attention`` with these arguments
    runs on this library, else (False, reason)."""
    if attn_mask is not None:
        return False, "an explicit attn_mask is not supported (use is_causal)"
    if dropout_p != 0.0:
        return False, "dropout is not supported"
    if enable_gqa:
        return False, "grouped-query attention is not supported"
    for name, t in (("query", query), ("key", key), ("value", value)):
        if not isinstance(t, torch.Tensor):
            return False, f"{name} is not a tensor"
        if t.device.type != "cuda":
            return False, f"{name} is not on a GPU"
        if t.dim() != 4:
            return False, f"{name} must be 4-D [B, H, seq, D]"
    if not (query.device == key.device == value.device):
        return False, "query, key and value are on different devices"
    if not (query.dtype == key.dtype == value.dtype):
        return False, "query, key and value have different dtypes"
    if query.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        return False, f"dtype {query.dtype} is not supported (float32, bfloat16 or float16)"
    B, H, M, D = query.shape
    if key.shape[:2] != (B, H) or key.shape[3] != D or value.shape[:3] != key.shape[:3]:
        return False, "key/value shapes do not match the query (same B, H; key's D; one N)"
    if D not in FWD_HEAD_DIMS:
        return False, f"head dim {D} is not supported ({FWD_HEAD_DIMS})"
    Dv = value.shape[3]
    if Dv != D and Dv not in FWD_HEAD_DIMS:
        return False, f"value head dim {Dv} is not supported ({FWD_HEAD_DIMS})"
    if M > 0 and key.shape[2] == 0:
        return False, "no keys"
    if scale is not None and not math.isfinite(float(scale)):
        return False, "scale is not finite"
    wants_grad = torch.is_grad_enabled() and any(
        t.requires_grad for t in (query, key, value))
    if wants_grad and Dv != D:
        return False, "the backward needs the value head dim equal to the query's"
    if wants_grad and (query.dtype not in BWD_DTYPES or D not in BWD_HEAD_DIMS):
        return False, (f"the backward supports bf16 and fp16 with head dim in {BWD_HEAD_DIMS} "
                       f"(inputs require grad)")
    return True, ""


def scaled_dot_product_attention(query, key, value, attn_mask=None, dropout_p: float = 0.0,
                                 is_causal: bool = False, scale: Optional[float] = None,
                                 enable_gqa: bool = False) -> torch.Tensor:
    """torch's SDPA signature on this library's kernels (raises
    NotImplementedError with the reason when they do not apply)."""
    ok, why = sdpa_checker(query, key, value, attn_mask, dropout_p, is_causal, scale,
                           enable_gqa)
    if not ok:
        raise NotImplementedError(f"scaled_dot_product_attention: {why}")
    return attention(query, key, value, is_causal=is_causal, scale=scale)


_SDPA_ARGS = ("query", "key", "value", "attn_mask", "dropout_p", "is_causal", "scale",
              "enable_gqa")
_SDPA_DEFAULTS = {"attn_mask": None, "dropout_p": 0.0, "is_causal": False, "scale": None,
                  "enable_gqa": False}


def _sdpa_call_args(args, kwargs) -> dict:
    """torch's SDPA arguments as one name -> value dict (positional or keyword)."""
    if len(args) > len(_SDPA_ARGS):
        raise TypeError("scaled_dot_product_attention: too many positional arguments")
    out = dict(_SDPA_DEFAULTS)
    out.update(zip(_SDPA_ARGS, args))
    for name, val in kwargs.items():
        if name not in _SDPA_ARGS:
            raise TypeError(f"scaled_dot_product_attention: unexpected argument {name!r}")
        out[name] = val
    return out


class route_sdpa(TorchFunctionMode):
    """While active, ``torch.nn.functional.scaled_dot_product_attention``
    calls run on this library when ``sdpa_checker`` accepts them.

    ``strict=True``: a rejected call raises NotImplementedError with the
    checker's reason. ``strict=False``: it runs torch's own SDPA instead.
    ``routed`` and ``declined`` count the calls of each kind. Every other
    torch function passes through unchanged. Calls that torch makes from
    inside another function that this mode sees first (for example the
    functional forward of ``nn.MultiheadAttention``) run with the mode
    suspended, as torch suspends a mode while its handler runs, and are not
    routed.
    """

    def __init__(self, strict: bool = True):
        super().__init__()
        self.strict = strict
        self.routed = 0
        self.declined = 0

    def __torch_function__(self, func, types, args=(), kwargs=None):
        kwargs = kwargs or {}
        if func is not torch.nn.functional.scaled_dot_product_attention:
            return func(*args, **kwargs)
        a = _sdpa_call_args(args, kwargs)
        ok, why = sdpa_checker(**a)
        if not ok:
            if self.strict:
                raise NotImplementedError(f"scaled_dot_product_attention: {why}")
            self.declined += 1
            return func(*args, **kwargs)
        self.routed += 1
        return attention(a["query"], a["key"], a["value"], is_causal=bool(a["is_causal"]),
                         scale=a["scale"])
