"""A torch autograd Linear layer over the library's quantizers and GEMMs.

Every product of the layer runs in the library's kernels (argument
marshalling only here): forward Y = X W^T, dgrad dX = dY W, wgrad dW = dY^T X,
with the operands quantized by the recipe:

  "blockwise"   1x128 tiles for X and dY, 128x128 blocks for W, online
                ("Can you explain the role of FP8 precision in DeepSeek-V3
                training", sections "Fine-grained quantization", "Online
                quantization"; E4M3 throughout, section "Unified E4M3 format")
  "per_tensor"  one current scale per tensor, E4M3 ("Accelerating FP8
                training performance with the NVIDIA NeMo framework",
                per-tensor recipe)
  "delayed"     per-tensor scales from an amax history, X and W in E4M3,
                dY in E5M2 (the hybrid recipe the DeepSeek page contrasts)

X is quantized once in the forward pass for both of its uses (row-wise for
Y, column-wise along the tokens for dW), W once for Y and dX, dY once in the
backward pass for dX and dW.  Y and dX are BF16, dW is FP32.  Shapes: the
token count and both feature counts must be multiples of 128.  fp8_mma=True
runs the three products on the FP8 matrix instructions (partial sums
promoted to FP32 per 128-deep block, section "Increasing accumulation
precision") instead of the exact FP16 decode.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import ops

RECIPES = ("blockwise", "per_tensor", "delayed")


class DelayedState:
    """Amax histories of one layer's X, W and dY for the delayed recipe."""

    def __init__(self, device, length: int = 16):
        self.length = length
        self.hist = {k: torch.zeros(length, dtype=torch.float32, device=device) for k in ("x", "w", "dy")}
        self.step = {k: 0 for k in ("x", "w", "dy")}

    def quantize(self, t: torch.Tensor, role: str, elem: str) -> ops.Quantized:
        slot = self.step[role] % self.length
        self.step[role] += 1
        return ops.quantize_delayed(t, self.hist[role], slot, elem, rowwise=True, colwise=True)


def _quant(t: torch.Tensor, role: str, recipe: str, state: Optional[DelayedState]) -> ops.Quantized:
    if recipe == "blockwise":
        return ops.quantize_blockwise(t, "block" if role == "w" else "tile", rowwise=True, colwise=True)
    if recipe == "per_tensor":
        return ops.quantize_blockwise(t, "tensor", rowwise=True, colwise=True)
    return state.quantize(t, role, "e5m2" if role == "dy" else "e4m3")


class _FP8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, recipe, state, fp8_mma):
        qx = _quant(x, "x", recipe, state)
        qw = _quant(w.to(torch.bfloat16).contiguous(), "w", recipe, state)
        y = ops.gemm_block_scaled(qx.rowwise(), qw.rowwise(), torch.bfloat16, fp8_mma=fp8_mma)
        ctx.qx, ctx.qw, ctx.recipe, ctx.state, ctx.fp8_mma = qx, qw, recipe, state, fp8_mma
        ctx.w_dtype = w.dtype
        return y

    @staticmethod
    def backward(ctx, dy):
        dy = dy.to(torch.bfloat16).contiguous()
        qdy = _quant(dy, "dy", ctx.recipe, ctx.state)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = ops.gemm_block_scaled(qdy.rowwise(), ctx.qw.colwise(), torch.bfloat16, fp8_mma=ctx.fp8_mma)
        if ctx.needs_input_grad[1]:
            dw = ops.gemm_block_scaled(qdy.colwise(), ctx.qx.colwise(), torch.float32,
                                       fp8_mma=ctx.fp8_mma).to(ctx.w_dtype)
        ctx.qx = ctx.qw = None
        return dx, dw, None, None, None


def fp8_linear(x: torch.Tensor, w: torch.Tensor, recipe: str = "blockwise",
               state: Optional[DelayedState] = None, fp8_mma: bool = False) -> torch.Tensor:
    """Y = X W^T with the recipe's scaled FP8 operands in forward and backward.
    x: [T x K] (any float dtype; cast to BF16), w: [N x K] (FP32 master or
    BF16; quantized from its BF16 cast, dW returned in w's dtype); returns
    BF16."""
    if recipe not in RECIPES:
        raise ValueError(f"recipe must be one of {RECIPES}")
    if recipe == "delayed" and state is None:
        raise ValueError("the delayed recipe needs a DelayedState")
    if x.dim() != 2 or w.dim() != 2 or x.shape[1] != w.shape[1]:
        raise ValueError("x must be [T x K] and w [N x K]")
    T, K = x.shape
    N = w.shape[0]
    if T % 128 or K % 128 or N % 128:
        raise ValueError(f"tokens ({T}), in ({K}) and out ({N}) features must be multiples of 128")
    return _FP8LinearFn.apply(x.to(torch.bfloat16).contiguous(), w, recipe, state, fp8_mma)


class Linear(torch.nn.Module):
    """Linear layer (no bias) whose products run on scaled FP8 operands.
    The weight is an FP32 master copy; its BF16 cast is quantized each step."""

    def __init__(self, in_features: int, out_features: int, recipe: str = "blockwise",
                 device=None, history: int = 16, fp8_mma: bool = False):
        super().__init__()
        if recipe not in RECIPES:
            raise ValueError(f"recipe must be one of {RECIPES}")
        self.recipe = recipe
        self.fp8_mma = fp8_mma
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, dtype=torch.float32, device=device))
        torch.nn.init.normal_(self.weight, std=in_features ** -0.5)
        self.state = DelayedState(self.weight.device, history) if recipe == "delayed" else None

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        shape = x.shape
        y = fp8_linear(x.reshape(-1, shape[-1]), self.weight, self.recipe, self.state, self.fp8_mma)
        return y.reshape(*shape[:-1], self.weight.shape[0])
