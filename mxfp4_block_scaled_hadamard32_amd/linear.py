"""Linear layer whose GEMMs run in MXFP4 (or MXFP8), one toggle per GEMM.

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

Two variants from the same page:
  * w_block / dy_block = 32 or 64 ("The fix, and its supporting cast"): W and / or dY are
    quantized once in square tiles, so the transposed product reads the same codes and scales
    (the tile's transposed copy) instead of a re-blocked quantization; X stays 1x32.
  * fmt = "mxfp8": the query / key projections in MXFP8, X and W in E4M3 and dY in E5M2.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import (MX_E4M3, MX_E5M2, MX_ROUND_RNE, MX_SCALE_FLOOR, mx_gemm_dgrad, mx_gemm_fprop,
               mx_gemm_mxfp8, mx_gemm_wgrad, mx_quantize, mx_quantize_2d_blocks,
               mx_quantize_mxfp8)


@dataclass
class QuantSpec:
    """Options of one operand quantization (as for mx_quantize)."""
    scale_rule: int = MX_SCALE_FLOOR
    round: int = MX_ROUND_RNE
    hadamard: int = 0
    sign_mask: int = 0


@dataclass
class MXLinearConfig:
    fprop: bool = True          # Fprop in MX format
    dgrad: bool = True          # Dgrad in MX format
    wgrad: bool = True          # Wgrad in MX format
    fprop_q: QuantSpec = field(default_factory=QuantSpec)
    dgrad_q: QuantSpec = field(default_factory=QuantSpec)
    wgrad_q: QuantSpec = field(default_factory=QuantSpec)
    fmt: str = "mxfp4"          # "mxfp4" or "mxfp8"
    w_block: int = 1            # 1 (1x32 along each GEMM's reduction axis), 32 or 64 (tiles)
    dy_block: int = 1           # the same for dY
    seed: int = 1234            # Philox key base of stochastic rounding; advanced every call

    def next_seeds(self) -> tuple[int, int, int]:
        """Distinct keys for the X, W and dY quantizations of one call."""
        s = self.seed
        self.seed += 3
        return s, s + 1, s + 2

    def check(self):
        if self.fmt not in ("mxfp4", "mxfp8"):
            raise ValueError("fmt must be 'mxfp4' or 'mxfp8'")
        if self.w_block not in (1, 32, 64) or self.dy_block not in (1, 32, 64):
            raise ValueError("w_block and dy_block must be 1, 32 or 64")
        if self.fmt == "mxfp8" and (self.w_block != 1 or self.dy_block != 1):
            raise ValueError("MXFP8 operands are 1x32 blocks")
        tiled = [q for q, on in ((self.fprop_q, self.w_block > 1), (self.dgrad_q, self.w_block > 1
                 or self.dy_block > 1), (self.wgrad_q, self.dy_block > 1)) if on]
        if any(q.hadamard for q in tiled):
            raise ValueError("tiles are quantized without the Hadamard rotation")
        # one tile quantization serves two GEMMs: their options must agree on it
        rule = lambda q: (q.scale_rule, q.round)  # noqa: E731
        if self.w_block > 1 and self.fprop and self.dgrad and rule(self.fprop_q) != rule(self.dgrad_q):
            raise ValueError("W tiles are shared by Fprop and Dgrad: fprop_q and dgrad_q must "
                             "have the same scale_rule and round")
        if self.dy_block > 1 and self.dgrad and self.wgrad and rule(self.dgrad_q) != rule(self.wgrad_q):
            raise ValueError("dY tiles are shared by Dgrad and Wgrad: dgrad_q and wgrad_q must "
                             "have the same scale_rule and round")

    def w_tile_spec(self) -> QuantSpec:
        """Options of W's tile quantization: Fprop's, or Dgrad's when Fprop is off."""
        return self.fprop_q if self.fprop else self.dgrad_q

    def dy_tile_spec(self) -> QuantSpec:
        """Options of dY's tile quantization: Dgrad's, or Wgrad's when Dgrad is off."""
        return self.dgrad_q if self.dgrad else self.wgrad_q


def _q(t: torch.Tensor, axis: int, spec: QuantSpec, seed: int, fp8: int | None = None):
    if fp8 is not None:
        return mx_quantize_mxfp8(t, fmt=fp8, axis=axis, scale_rule=spec.scale_rule,
                                 round=spec.round, hadamard=spec.hadamard,
                                 sign_mask=spec.sign_mask, seed=seed)
    return mx_quantize(t, axis=axis, scale_rule=spec.scale_rule, round=spec.round,
                       hadamard=spec.hadamard, sign_mask=spec.sign_mask, seed=seed)


def _tiles(t: torch.Tensor, block: int, spec: QuantSpec, seed: int):
    """(codes, scales, codes_t, scales_t) of block x block tiles; scale granularity = block."""
    return mx_quantize_2d_blocks(t, block=block, scale_rule=spec.scale_rule, round=spec.round,
                                 seed=seed)


def _alpha(spec: QuantSpec) -> int:
    # two operands rotated with the same unnormalised transform along K: factor 32 -> 2^-5
    return -5 if spec.hadamard else 0


class MXLinearFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x: torch.Tensor, w: torch.Tensor, cfg: MXLinearConfig):
        cfg.check()
        sx, sw, sdy = cfg.next_seeds()
        ctx.cfg, ctx.seeds = cfg, (sx, sw, sdy)
        ctx.save_for_backward(x, w)
        ctx.w_tiles = None
        if not cfg.fprop:
            if cfg.dgrad and cfg.w_block > 1:
                ctx.w_tiles = _tiles(w, cfg.w_block, cfg.w_tile_spec(), sw)
            return x @ w.t()
        spec = cfg.fprop_q
        if cfg.fmt == "mxfp8":
            xq, xs = _q(x, 1, spec, sx, MX_E4M3)
            wq, ws = _q(w, 1, spec, sw, MX_E4M3)
            return mx_gemm_mxfp8(xq, xs, MX_E4M3, wq, ws, MX_E4M3, alpha_exp=_alpha(spec),
                                 out_dtype=x.dtype)
        xq, xs = _q(x, 1, spec, sx)
        if cfg.w_block > 1:
            ctx.w_tiles = _tiles(w, cfg.w_block, cfg.w_tile_spec(), sw)
            wq, ws, gw = ctx.w_tiles[0], ctx.w_tiles[1], cfg.w_block
        else:
            (wq, ws), gw = _q(w, 1, spec, sw), 1
        return mx_gemm_fprop(xq, xs, 1, wq, ws, gw, alpha_exp=_alpha(spec), out_dtype=x.dtype)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, w = ctx.saved_tensors
        cfg = ctx.cfg
        sx, sw, sdy = ctx.seeds
        dy = dy.contiguous().to(x.dtype)
        fp8 = cfg.fmt == "mxfp8"
        dx = dw = None
        dy_tiles = None
        if cfg.dy_block > 1 and not fp8 and (cfg.dgrad or cfg.wgrad):
            dy_tiles = _tiles(dy, cfg.dy_block, cfg.dy_tile_spec(), sdy)
        if ctx.needs_input_grad[0]:
            if cfg.dgrad:
                spec = cfg.dgrad_q
                if fp8:
                    dyq, dys = _q(dy, 1, spec, sdy, MX_E5M2)
                    wtq, wts = _q(w, 0, spec, sw, MX_E4M3)
                    dx = mx_gemm_mxfp8(dyq, dys, MX_E5M2, wtq, wts, MX_E4M3,
                                       alpha_exp=_alpha(spec), out_dtype=x.dtype)
                else:
                    if dy_tiles is not None:
                        dyq, dys, gdy = dy_tiles[0], dy_tiles[1], cfg.dy_block
                    else:
                        (dyq, dys), gdy = _q(dy, 1, spec, sdy), 1
                    if ctx.w_tiles is not None:
                        wtq, wts, gwt = ctx.w_tiles[2], ctx.w_tiles[3], cfg.w_block
                    else:
                        (wtq, wts), gwt = _q(w, 0, spec, sw), 1
                    dx = mx_gemm_dgrad(dyq, dys, gdy, wtq, wts, gwt, alpha_exp=_alpha(spec),
                                       out_dtype=x.dtype)
            else:
                dx = dy @ w
        if ctx.needs_input_grad[1]:
            if cfg.wgrad:
                spec = cfg.wgrad_q
                if fp8:
                    dytq, dyts = _q(dy, 0, spec, sdy, MX_E5M2)
                    xtq, xts = _q(x, 0, spec, sx, MX_E4M3)
                    dw = mx_gemm_mxfp8(dytq, dyts, MX_E5M2, xtq, xts, MX_E4M3,
                                       alpha_exp=_alpha(spec), out_dtype=w.dtype)
                else:
                    if dy_tiles is not None:
                        dytq, dyts, gdy = dy_tiles[2], dy_tiles[3], cfg.dy_block
                    else:
                        (dytq, dyts), gdy = _q(dy, 0, spec, sdy), 1
                    xtq, xts = _q(x, 0, spec, sx)
                    dw = mx_gemm_wgrad(dytq, dyts, gdy, xtq, xts, 1, alpha_exp=_alpha(spec),
                                       out_dtype=w.dtype)
            else:
                dw = dy.t() @ x
        ctx.w_tiles = None
        return dx, dw, None


class MXLinear(torch.nn.Module):
    """y = x W^T with the products in MX formats per MXLinearConfig (no bias). x: [T][K] bf16 with
    T and K multiples of 32 (of 128 for MXFP8, of the tile edge for tiled operands); W: [N][K]
    bf16 with N a multiple of 32 (128, tile edge)."""

    def __init__(self, in_features: int, out_features: int, cfg: MXLinearConfig | None = None,
                 device="cuda", dtype=torch.bfloat16):
        super().__init__()
        self.cfg = cfg or MXLinearConfig()
        w = torch.empty((out_features, in_features), device=device, dtype=dtype)
        torch.nn.init.normal_(w, std=in_features ** -0.5)
        self.weight = torch.nn.Parameter(w)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return MXLinearFunction.apply(x, self.weight, self.cfg)
