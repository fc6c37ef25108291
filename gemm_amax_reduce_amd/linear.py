"""NVFP4 linear layer over the C ABI: forward and backward of y = x W^T with
every product on the block-scaled NVFP4 GEMM.

The recipe follows the pages: [P4] aisight.pl "Koniec marnowania mocy ...",
section "Technologie stabilizujace proces treningowy" (stochastic rounding of
the gradients, the 16-point random Hadamard transform on the weight-gradient
operands, a share of the last layers kept in BF16) and [P3]
aibuzzwire.news "End-to-End 4-Bit Training", section "Unterschiedliche
Phasen, unterschiedliche Regeln" (nearest rounding in the forward pass,
stochastic rounding of the gradients).

    forward  y  = x W^T    A = x (axis 1, RNE),  B = W (axis 1, RNE)
    backward dx = dy W     A = dy (axis 1, SR),  B = W (axis 0, RNE)
             dW = dy^T x   A = dy (axis 0, RHT, SR), B = x (axis 0, RHT, RNE)

Each operand is read once for both of its layouts: x and W through
dual-layout calls in the forward pass (when their gradients are needed), dy
in the backward pass.  The backward keeps only the quantized operands, not x
and W.  The two operands of the weight gradient share one sign mask, so the
transform cancels in the product.  Every quantization and GEMM runs in the
HIP library; there is no CPU path.
"""
from __future__ import annotations

import torch

from . import (nvfp4_gemm_ws, nvfp4_quantize, nvfp4_quantize_dual, NVFP4Error)


def _out_dtype(t: torch.Tensor) -> torch.dtype:
    return torch.bfloat16 if t.dtype == torch.bfloat16 else torch.float32


class NVFP4LinearFunction(torch.autograd.Function):
    """y = x W^T for x [tokens, in], W [out, in]; returns y in x's dtype."""

    @staticmethod
    def forward(ctx, x, weight, seed: int, offset: int, sign_mask: int):
        if x.dim() != 2 or weight.dim() != 2 or x.shape[1] != weight.shape[1]:
            raise NVFP4Error("x must be [tokens, in] and weight [out, in]")
        x = x.contiguous()
        weight = weight.contiguous()
        need_dx, need_dw = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        # x along its rows for y and, transformed, along its columns for dW;
        # W along its rows for y and along its columns for dx
        qx0 = qw0 = None
        if need_dw:
            qx, qx0 = nvfp4_quantize_dual(x, rht0=True, sign_mask0=sign_mask)
        else:
            qx = nvfp4_quantize(x, axis=1)
        if need_dx:
            qw, qw0 = nvfp4_quantize_dual(weight)
        else:
            qw = nvfp4_quantize(weight, axis=1)
        y = nvfp4_gemm_ws(qx, qw, _out_dtype(x))
        if y.dtype != x.dtype:
            y = y.to(x.dtype)
        ctx.qx0, ctx.qw0 = qx0, qw0
        ctx.x_dtype, ctx.w_dtype = x.dtype, weight.dtype
        ctx.seed, ctx.offset, ctx.sign_mask = seed, offset, sign_mask
        return y

    @staticmethod
    def backward(ctx, dy):
        dy = dy.contiguous().to(ctx.x_dtype)
        # dy along its columns (data gradient) and, transformed, along its
        # rows (weight gradient); distinct Philox offsets keep the two draws
        # independent
        qdy1, qdy0 = nvfp4_quantize_dual(dy, rounding1="sr", seed1=ctx.seed, offset1=2 * ctx.offset,
                                         rht0=True, sign_mask0=ctx.sign_mask, rounding0="sr", seed0=ctx.seed,
                                         offset0=2 * ctx.offset + 1)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            dx = nvfp4_gemm_ws(qdy1, ctx.qw0, _out_dtype(dy))
            if dx.dtype != ctx.x_dtype:
                dx = dx.to(ctx.x_dtype)
        if ctx.needs_input_grad[1]:
            dw = nvfp4_gemm_ws(qdy0, ctx.qx0, torch.bfloat16 if ctx.w_dtype == torch.bfloat16 else torch.float32)
            if dw.dtype != ctx.w_dtype:
                dw = dw.to(ctx.w_dtype)
        ctx.qx0 = ctx.qw0 = None
        return dx, dw, None, None, None


class NVFP4Linear(torch.nn.Module):
    """Bias-free linear layer whose products run in NVFP4.

    keep_bf16=True runs the layer as a plain bf16 linear instead: the pages
    keep a share of the final layers in BF16 (the caller decides which).
    Each forward call draws a fresh Philox offset, so successive steps use
    independent stochastic rounding.
    """

    def __init__(self, in_features: int, out_features: int, seed: int = 0, sign_mask: int = 0xA5C3,
                 keep_bf16: bool = False, device=None, dtype=torch.bfloat16):
        super().__init__()
        if in_features % 16 or out_features % 16:
            raise NVFP4Error("in_features and out_features must be multiples of 16")
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, device=device, dtype=dtype))
        torch.nn.init.normal_(self.weight, std=0.02)
        self.seed, self.sign_mask, self.keep_bf16 = seed, sign_mask & 0xFFFF, keep_bf16
        self._calls = 0

    def forward(self, x):
        """x [..., in] -> [..., out]; the leading dimensions are the tokens."""
        if self.keep_bf16:
            return torch.nn.functional.linear(x.to(torch.bfloat16), self.weight.to(torch.bfloat16)).to(x.dtype)
        if x.dim() < 1 or x.shape[-1] != self.weight.shape[1]:
            raise NVFP4Error(f"x must end in {self.weight.shape[1]} features, got shape {tuple(x.shape)}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1])
        if x2.shape[0] % 16:
            raise NVFP4Error("the token count must be a multiple of 16 (the weight gradient reduces over it)")
        offset = self._calls
        self._calls += 1
        y = NVFP4LinearFunction.apply(x2, self.weight, self.seed, offset, self.sign_mask)
        return y.reshape(*lead, self.weight.shape[0])
