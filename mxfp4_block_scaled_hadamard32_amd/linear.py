"""Linear layer whose GEMMs run in MXFP4, one toggle per GEMM.

"Pretraining large language models with MXFP4" (abstract) enables FP4 progressively in the
forward product (Fprop), the activation gradient (Dgrad) and the weight gradient (Wgrad) of
every linear layer; "Stable FP4 Training via Transposition-Invariant Block Quantization"
("The aha: transposition scrambles the blocks") gives the three products and the axis each
one reduces over. This autograd function quantizes each operand along the reduction axis of
the GEMM that consumes it and calls the library's GEMMs; the quantizers are treated as the
identity in the backward pass (straight-through). A GEMM whose toggle is off is the bf16
product, the comparison arm of that progressive enabling.

    Fprop  Y  [T][N] = X [T][K] W [N][K]^T     X, W along K
    Dgrad  dX [T][K] = dY[T][N] W [N][K]       dY along N, W along N (K-major copy of W^T)
    Wgrad  dW [N][K] = dY^T X                  dY and X along T (K-major copies of dY^T, X^T)
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import (MX_ROUND_RNE, MX_SCALE_FLOOR, mx_gemm_dgrad, mx_gemm_fprop, mx_gemm_wgrad,
               mx_quantize)


@dataclass
class QuantSpec:
    """Options of one operand quantization (as for mx_quantize)."""
    scale_rule: int = MX_SCALE_FLOOR
    round: int = MX_ROUND_RNE
    hadamard: int = 0
    sign_mask: int = 0


@dataclass
class MXLinearConfig:
    fprop: bool = True          # Fprop in MXFP4
    dgrad: bool = True          # Dgrad in MXFP4
    wgrad: bool = True          # Wgrad in MXFP4
    fprop_q: QuantSpec = field(default_factory=QuantSpec)
    dgrad_q: QuantSpec = field(default_factory=QuantSpec)
    wgrad_q: QuantSpec = field(default_factory=QuantSpec)
    seed: int = 1234            # Philox key base of stochastic rounding; advanced every call

    def next_seeds(self) -> tuple[int, int, int]:
        """Distinct keys for the X, W and dY quantizations of one call."""
        s = self.seed
        self.seed += 3
        return s, s + 1, s + 2


def _q(t: torch.Tensor, axis: int, spec: QuantSpec, seed: int):
    return mx_quantize(t, axis=axis, scale_rule=spec.scale_rule, round=spec.round,
                       hadamard=spec.hadamard, sign_mask=spec.sign_mask, seed=seed)


def _alpha(spec: QuantSpec) -> int:
    # two operands rotated with the same unnormalised transform along K: factor 32 -> 2^-5
    return -5 if spec.hadamard else 0


class MXLinearFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, cfg: MXLinearConfig):
        sx, sw, sdy = cfg.next_seeds()
        ctx.cfg, ctx.seeds = cfg, (sx, sw, sdy)
        ctx.save_for_backward(x, w)
        if cfg.fprop:
            xq, xs = _q(x, 1, cfg.fprop_q, sx)
            wq, ws = _q(w, 1, cfg.fprop_q, sw)
            return mx_gemm_fprop(xq, xs, 1, wq, ws, 1, alpha_exp=_alpha(cfg.fprop_q),
                                 out_dtype=x.dtype)
        return x @ w.t()

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, w = ctx.saved_tensors
        cfg = ctx.cfg
        sx, sw, sdy = ctx.seeds
        dy = dy.contiguous().to(x.dtype)
        dx = dw = None
        if ctx.needs_input_grad[0]:
            if cfg.dgrad:
                dyq, dys = _q(dy, 1, cfg.dgrad_q, sdy)
                wtq, wts = _q(w, 0, cfg.dgrad_q, sw)
                dx = mx_gemm_dgrad(dyq, dys, 1, wtq, wts, 1, alpha_exp=_alpha(cfg.dgrad_q),
                                   out_dtype=x.dtype)
            else:
                dx = dy @ w
        if ctx.needs_input_grad[1]:
            if cfg.wgrad:
                dytq, dyts = _q(dy, 0, cfg.wgrad_q, sdy)
                xtq, xts = _q(x, 0, cfg.wgrad_q, sx)
                dw = mx_gemm_wgrad(dytq, dyts, 1, xtq, xts, 1, alpha_exp=_alpha(cfg.wgrad_q),
                                   out_dtype=w.dtype)
            else:
                dw = dy.t() @ x
        return dx, dw, None


class MXLinear(torch.nn.Module):
    """y = x W^T with the products in MXFP4 per MXLinearConfig (no bias). x: [T][K] bf16 with T
    and K multiples of 32; W: [N][K] bf16 with N a multiple of 32."""

    def __init__(self, in_features: int, out_features: int, cfg: MXLinearConfig | None = None,
                 device="cuda", dtype=torch.bfloat16):
        super().__init__()
        self.cfg = cfg or MXLinearConfig()
        w = torch.empty((out_features, in_features), device=device, dtype=dtype)
        torch.nn.init.normal_(w, std=in_features ** -0.5)
        self.weight = torch.nn.Parameter(w)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return MXLinearFunction.apply(x, self.weight, self.cfg)
