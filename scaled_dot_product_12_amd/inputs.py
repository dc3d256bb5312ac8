"""Seeded synthetic inputs for the attention forward workloads.

This module holds no attention arithmetic: it only draws tensors and rearranges
them. Both the HIP path's tests/benchmark and the CPU oracle are fed from here.

Recipe (every workload): ``g = torch.Generator("cpu").manual_seed(seed)``, then
Q, K, V in that order, each ``torch.randn(shape, dtype=float32, generator=g)``.
bf16 (fp16, fp8) workloads round those fp32 draws with ``.to(torch.bfloat16)``
(``.to(torch.float16)``, ``.to(torch.float8_e4m3fn)``), round-to-nearest-even. The upstream gradient dO of a backward problem is
drawn the same way from its own generator, seeded with ``seed + DOUT_SEED_OFFSET``
(so Q, K, V are the same draws as the forward problem's). Shapes follow the
pages' workloads:

* "Extend Thunder with CUDA-Python": Q, K, V of shape (96, 512, 128), fp32.
* "Blackwell Attention Example", test harness: bf16 (z, h, n_ctx, head_dim)
  tensors at long context.
* The PopcornBench axial-attention trajectory: images of 32x32 tokens, model
  dim 64 split into 4 heads of 16, attended first along rows and then along
  columns (128 sequences of length 32 per pass at batch 4). The problem's own
  input files are not available, so i.i.d. N(0, 1) tensors of that shape stand
  in for the projected per-head Q, K, V.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    """One attention forward problem: shapes, dtype, masking, seed."""
    name: str
    B: int
    H: int
    M: int
    N: int
    D: int
    dtype: str            # "fp32", "bf16", "fp16" or "fp8" (e4m3 inputs, bf16 output)
    causal: bool
    seed: int
    axial: str = ""       # "" or "row" / "col" / "both" for the axial passes
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """1/sqrt(D) rounded to fp32, the value handed to the kernel."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    @property
    def flops(self) -> float:
        """4*B*H*M*N*D, halved when causal (the pages' counting convention)."""
        f = 4.0 * self.B * self.H * self.M * self.N * self.D
        return f / 2 if self.causal else f

    def algorithmic_bytes(self) -> int:
        """Read Q, K, V once; write O once (the input dtype; bf16 for fp8
        inputs) and L once (fp32)."""
        es_in = {"fp32": 4, "bf16": 2, "fp16": 2, "fp8": 1}[self.dtype]
        es_out = 2 if self.dtype == "fp8" else es_in
        return (self.B * self.H * (es_in * (self.M + 2 * self.N) * self.D
                                   + es_out * self.M * self.D)
                + 4 * self.B * self.H * self.M)

    def describe(self) -> str:
        c = "causal" if self.causal else "non-causal"
        ax = f" axial-{self.axial}" if self.axial else ""
        return (f"{self.dtype}{ax} B={self.B} H={self.H} M={self.M} N={self.N} "
                f"D={self.D} {c}")


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", 1, 1, 128, 128, 64, "fp32", False, 1,
                   note="single head fp32"),
    "c2": Workload("c2", 96, 1, 512, 512, 128, "fp32", False, 2,
                   note="page-1 notebook batch of 96, fp32"),
    "c2c": Workload("c2c", 96, 1, 512, 512, 128, "fp32", True, 2,
                    note="same tensors as c2, causal"),
    "c3r": Workload("c3r", 128, 4, 32, 32, 16, "fp32", False, 3, axial="row",
                    note="axial row pass: 4 images x 32 rows"),
    "c3c": Workload("c3c", 128, 4, 32, 32, 16, "fp32", False, 3, axial="col",
                    note="axial column pass: 4 images x 32 columns"),
    # Both passes in one launch: the row gather and the column gather of the
    # same image tensors stacked along the batch ([256, 4, 32, 16]); the two
    # passes are independent once Q, K and V are gathered.
    "c3": Workload("c3", 256, 4, 32, 32, 16, "fp32", False, 3, axial="both",
                   note="axial row and column passes in one launch"),
    "c4": Workload("c4", 4, 16, 4096, 4096, 128, "bf16", False, 4,
                   note="long-sequence bf16"),
    "c5": Workload("c5", 2, 32, 8192, 8192, 128, "bf16", True, 5,
                   note="causal bf16, longer context"),
    # The bench shapes of "Blackwell Attention Example" (main function):
    # (z, h, n_ctx, head_dim) = (4, 32, 8192, 64) and (4, 32, 8192, 128),
    # bf16, non-causal.
    "p64": Workload("p64", 4, 32, 8192, 8192, 64, "bf16", False, 6,
                    note="Blackwell example bench shape, head dim 64"),
    "p128": Workload("p128", 4, 32, 8192, 8192, 128, "bf16", False, 7,
                     note="Blackwell example bench shape, head dim 128"),
    # The long-sequence shape in fp16 (the Blackwell example's main function
    # describes its test as float16): the same draws as c4, rounded to fp16.
    "c4h": Workload("c4h", 4, 16, 4096, 4096, 128, "fp16", False, 4,
                    note="long-sequence fp16"),
    # The long-sequence shape with fp8 (e4m3) inputs and P rounded to fp8 for
    # the second product (the Blackwell example casts P to the value dtype):
    # c4's draws rounded to e4m3; V is handed to the kernel transposed.
    "c4f8": Workload("c4f8", 4, 16, 4096, 4096, 128, "fp8", False, 4,
                     note="long-sequence fp8 e4m3"),
}

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16,
       "fp8": torch.float8_e4m3fn}


def make_qkv(B: int, H: int, M: int, N: int, D: int, dtype: str = "fp32",
             seed: int = 0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Q [B,H,M,D], K [B,H,N,D], V [B,H,N,D] on the CPU, contiguous."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, M, D), dtype=torch.float32, generator=g)
    k = torch.randn((B, H, N, D), dtype=torch.float32, generator=g)
    v = torch.randn((B, H, N, D), dtype=torch.float32, generator=g)
    if dtype != "fp32":
        q, k, v = (t.to(_DT[dtype]) for t in (q, k, v))
    return q, k, v


DOUT_SEED_OFFSET = 7919


def make_dout(B: int, H: int, M: int, D: int, dtype: str = "fp32",
              seed: int = 0) -> torch.Tensor:
    """Upstream gradient dO [B,H,M,D] on the CPU, contiguous."""
    g = torch.Generator("cpu").manual_seed(seed + DOUT_SEED_OFFSET)
    t = torch.randn((B, H, M, D), dtype=torch.float32, generator=g)
    return t if dtype == "fp32" else t.to(_DT[dtype])


# Axial images: 4 images of 32 x 32 tokens, 4 heads of dim 16.
AXIAL_IMAGES, AXIAL_H, AXIAL_W, AXIAL_HEADS, AXIAL_HD = 4, 32, 32, 4, 16


def make_axial(seed: int = 3):
    """Per-head image tensors (b, y, x, head, hd) for Q, K, V, fp32, CPU."""
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (AXIAL_IMAGES, AXIAL_H, AXIAL_W, AXIAL_HEADS, AXIAL_HD)
    return tuple(torch.randn(shape, dtype=torch.float32, generator=g)
                 for _ in range(3))


def axial_rows(t: torch.Tensor) -> torch.Tensor:
    """Row pass gather: (b, y, x, head, hd) -> [(b*y), head, x, hd] contiguous."""
    b, y, x, h, d = t.shape
    return t.permute(0, 1, 3, 2, 4).reshape(b * y, h, x, d).contiguous()


def axial_cols(t: torch.Tensor) -> torch.Tensor:
    """Column pass gather: (b, y, x, head, hd) -> [(b*x), head, y, hd] contiguous."""
    b, y, x, h, d = t.shape
    return t.permute(0, 2, 3, 1, 4).reshape(b * x, h, y, d).contiguous()


def workload_inputs(w: Workload):
    """The seeded CPU tensors (q, k, v) for a named workload."""
    if w.axial:
        qi, ki, vi = make_axial(w.seed)
        if w.axial == "both":
            return tuple(torch.cat([axial_rows(t), axial_cols(t)], 0).contiguous()
                         for t in (qi, ki, vi))
        f = axial_rows if w.axial == "row" else axial_cols
        return f(qi), f(ki), f(vi)
    return make_qkv(w.B, w.H, w.M, w.N, w.D, w.dtype, w.seed)


# The fused axial block: an image tensor x [B, Hh, W, C] and the weights of the
# row pass and of the column pass, each (ln_w [C], ln_b [C], w_qkv [3C, C],
# w_out [C, C], b_out [C]). Draw order from one generator: x ~ N(0, 1), then
# for the row pass and then the column pass: ln_w = 1 + 0.1 N(0, 1),
# ln_b = 0.1 N(0, 1), and w_qkv, w_out, b_out ~ U(-1/sqrt(C), 1/sqrt(C))
# (torch's default initialisation of its linear layers; the LayerNorm affine is
# perturbed from its default of (1, 0) so that both terms matter).
AXIAL_BLOCK_SEED = 6


def make_axial_block(B: int = AXIAL_IMAGES, Hh: int = AXIAL_H, W: int = AXIAL_W,
                     C: int = AXIAL_HEADS * AXIAL_HD, seed: int = AXIAL_BLOCK_SEED):
    """(x, row_params, col_params) as fp32 CPU tensors."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn((B, Hh, W, C), dtype=torch.float32, generator=g)
    bound = 1.0 / math.sqrt(C)

    def uniform(shape):
        return (torch.rand(shape, dtype=torch.float32, generator=g) * 2.0 - 1.0) * bound

    def pass_params():
        ln_w = 1.0 + 0.1 * torch.randn((C,), dtype=torch.float32, generator=g)
        ln_b = 0.1 * torch.randn((C,), dtype=torch.float32, generator=g)
        return (ln_w, ln_b, uniform((3 * C, C)), uniform((C, C)), uniform((C,)))

    row = pass_params()
    return x, row, pass_params()
