"""Float8Linear: a Linear layer whose GEMMs run in FP8 on the library's kernels.

The layer is one autograd node with a hand-written backward, as in "FP8
Training: Quantization, Autograd, Torchao", section 6: the quantization and
the scaled GEMMs are not recorded op by op. Forward and backward are single
calls of the C ABI (fp8_linear_fwd / fp8_linear_bwd), so every step of the
math runs in this package's HIP kernels; this module only allocates outputs
and workspaces and reshapes.

Recipes ("FP8 training on AMD GPUs with TorchTitan and TorchAO", Figure 1
caption):
  - "rowwise": per-row e4m3 scales for x and w in the forward, e5m2 per row
    for grad_out, w per column for grad-input, grad-weight in BF16;
  - "tensorwise": one scale per tensor, all three GEMMs in FP8 (the
    grad-weight GEMM takes grad_out and x transposed, written by one dual
    quantization launch); needs a multiple of 16 rows.

What the backward keeps: the bf16 input and weight (references, no copy).
The kernels write every FP8 operand in the layout its GEMM reads straight
from bf16, so the backward re-quantizes instead of transposing FP8 copies
saved by the forward; a deterministic quantizer gives the forward's bytes.
"""
from __future__ import annotations

import math

import torch

from . import (OUT_BF16, RECIPE_ROWWISE_BF16_WGRAD, RECIPE_TENSORWISE, fp8_linear_bwd, fp8_linear_fwd,
               fp8_linear_ws_bytes, load)

_RECIPES = {"rowwise": RECIPE_ROWWISE_BF16_WGRAD, "tensorwise": RECIPE_TENSORWISE}


def _check_operand(t: torch.Tensor, name: str):
    if t.device.type != "cuda":
        raise RuntimeError(f"Float8Linear: {name} must be on a ROCm GPU (got {t.device})")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"Float8Linear: {name} must be bfloat16 (got {t.dtype})")


class Float8LinearFunction(torch.autograd.Function):
    """y = x w^T through fp8_linear_fwd; grad_x, grad_w through fp8_linear_bwd.
    x [..., K] and w [N, K] bf16 on the GPU; y [..., N] bf16."""

    @staticmethod
    def forward(ctx, x, weight, recipe: int, eps: float):
        _check_operand(x, "input")
        _check_operand(weight, "weight")
        K = x.shape[-1]
        N = weight.shape[0]
        if weight.shape[1] != K:
            raise ValueError(f"Float8Linear: input has {K} features, weight expects {weight.shape[1]}")
        x2 = x.reshape(-1, K).contiguous()
        w = weight.contiguous()
        M = x2.shape[0]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
        ws = torch.empty(fp8_linear_ws_bytes(M, N, K, recipe), dtype=torch.uint8, device=x.device)
        fp8_linear_fwd(x2, w, recipe, eps, OUT_BF16, y, ws)
        ctx.save_for_backward(x2, w)
        ctx.recipe, ctx.eps, ctx.x_shape = recipe, eps, x.shape
        return y.reshape(*x.shape[:-1], N)

    @staticmethod
    def backward(ctx, grad_out):
        x2, w = ctx.saved_tensors
        M, K = x2.shape
        N = w.shape[0]
        gy = grad_out.reshape(-1, N)
        if gy.dtype != torch.bfloat16:
            gy = gy.to(torch.bfloat16)
        gy = gy.contiguous()
        gx = torch.empty((M, K), dtype=torch.bfloat16, device=x2.device)
        gw = torch.empty((N, K), dtype=torch.bfloat16, device=x2.device)
        ws = torch.empty(fp8_linear_ws_bytes(M, N, K, ctx.recipe), dtype=torch.uint8, device=x2.device)
        fp8_linear_bwd(gy, x2, w, ctx.recipe, ctx.eps, gx, gw, ws)
        return gx.reshape(ctx.x_shape), gw, None, None


class Float8Linear(torch.nn.Module):
    """Drop-in Linear (bf16 parameters) whose matmuls run in FP8.

    in_features must be a multiple of 16 and out_features a multiple of 16
    (the FP8 GEMM's contraction and the backward's column quantization); the
    tensorwise recipe also needs a multiple of 16 rows in the flattened
    input. The bias, if any, is added in bf16 after the FP8 GEMM."""

    def __init__(self, in_features: int, out_features: int, bias: bool = False, recipe: str = "rowwise",
                 eps: float = 1e-12, device=None):
        super().__init__()
        if recipe not in _RECIPES:
            raise ValueError(f"recipe must be one of {sorted(_RECIPES)}")
        self.in_features, self.out_features = in_features, out_features
        self.recipe, self.eps = recipe, float(eps)
        kw = dict(dtype=torch.bfloat16, device=device)
        self.weight = torch.nn.Parameter(torch.empty((out_features, in_features), **kw))
        self.bias = torch.nn.Parameter(torch.empty(out_features, **kw)) if bias else None
        self.reset_parameters()

    def reset_parameters(self):
        # the default initialization of torch.nn.Linear
        torch.nn.init.kaiming_uniform_(self.weight, a=math.sqrt(5))
        if self.bias is not None:
            bound = 1 / math.sqrt(self.in_features) if self.in_features > 0 else 0
            torch.nn.init.uniform_(self.bias, -bound, bound)

    @classmethod
    def from_linear(cls, linear: torch.nn.Linear, recipe: str = "rowwise", eps: float = 1e-12):
        """A Float8Linear holding a bf16 copy of `linear`'s parameters."""
        m = cls(linear.in_features, linear.out_features, bias=linear.bias is not None, recipe=recipe, eps=eps,
                device=linear.weight.device)
        with torch.no_grad():
            m.weight.copy_(linear.weight.to(torch.bfloat16))
            if linear.bias is not None:
                m.bias.copy_(linear.bias.to(torch.bfloat16))
        return m

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        load()
        y = Float8LinearFunction.apply(x, self.weight, _RECIPES[self.recipe], self.eps)
        return y if self.bias is None else y + self.bias

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bias={self.bias is not None}, recipe={self.recipe}")
