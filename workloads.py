"""Seeded synthetic inputs of the five workloads (shared by the tests, the benchmark and smoke).

This module holds input generation only — no quantization, transform or GEMM arithmetic — so
both the GPU path and the CPU oracle can consume the same tensors without sharing method code.

Shapes and value distributions follow the workloads the pages train on (Llama-3.1-8B MLP and a
70B dense model, one GPU's share of tokens); no dataset or trained weight is used:
  tiny        X, W 256x256 fp32 ~ N(0,1), 4 random columns of X scaled x50
  quant       A 8192x4096 bf16 ~ Student-t(3), 0.5% of channels (20 columns) scaled x100
  llama8b_up  X 8192x4096 ~ t(3), W 14336x4096 ~ N(0, 0.02), dY 8192x14336 ~ 1e-3 N(0,1) * rho_t
              with a per-row factor rho_t = |t(3)| (heavy-tailed rows)
  blocks_2d   W 14336x4096 and dY 8192x14336 ~ t(3) with 0.5% of columns x100, X 8192x4096 ~ t(3)
  llama70b_dn H 16384x28672 ~ t(3), W 8192x28672 ~ N(0, 0.01), dY 16384x8192 ~ N(0, 1e-3)
Student-t(3) is drawn as Z / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from independent normals.

Random quantities the method itself consumes (the +/-1 sign mask of the randomized Hadamard
transform, the stochastic-rounding seed) are produced here too and handed to both sides.
"""
from __future__ import annotations

import numpy as np
import torch

SR_SEED = 1234  # Philox key of every stochastic rounding in the workloads


def sign_mask(seed: int = SR_SEED) -> int:
    """32-bit random +/-1 diagonal (bit j set = negate block position j), from numpy's PCG64."""
    return int(np.random.default_rng(seed).integers(0, 1 << 32, dtype=np.uint64))


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def student_t3(shape, seed: int, device="cpu", chunk_rows: int = 2048) -> torch.Tensor:
    """float32 Student-t with 3 degrees of freedom, generated in row chunks to bound memory."""
    g = _gen(seed, device)
    rows, cols = shape
    out = torch.empty(shape, dtype=torch.float32, device=device)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = torch.randn((4, r1 - r0, cols), generator=g, device=device, dtype=torch.float32)
        chi = (z[1] * z[1] + z[2] * z[2] + z[3] * z[3]) / 3.0
        out[r0:r1] = z[0] / torch.sqrt(chi)
    return out


def normal(shape, std: float, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def outlier_columns(x: torch.Tensor, count: int, factor: float, seed: int) -> torch.Tensor:
    """Scales `count` distinct random columns of x by `factor` (outlier channels)."""
    rng = np.random.default_rng(seed)
    cols = rng.choice(x.shape[1], size=count, replace=False)
    idx = torch.as_tensor(np.sort(cols), device=x.device)
    x[:, idx] *= factor
    return x


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """Host uint16 bit patterns of a bf16 tensor (the oracle's bf16 input form)."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(x: torch.Tensor) -> np.ndarray:
    return np.ascontiguousarray(x.detach().float().cpu().numpy())


def host_input(x: torch.Tensor) -> np.ndarray:
    """The oracle's view of a GPU-path input: uint16 bits for bf16, float32 otherwise."""
    return bf16_bits(x) if x.dtype == torch.bfloat16 else host_f32(x)


# ------------------------------------------------------------------------------------------------
# the five workloads
# ------------------------------------------------------------------------------------------------
def tiny(device="cpu"):
    """X, W 256x256 fp32 ~ N(0,1) (seed 0); 4 random columns of X x50."""
    X = normal((256, 256), 1.0, seed=0, device=device)
    W = normal((256, 256), 1.0, seed=1, device=device)
    outlier_columns(X, 4, 50.0, seed=0)
    return {"X": X, "W": W}


def quant_stream(device="cpu", rows: int = 8192, cols: int = 4096):
    """Activation 8192x4096 bf16 ~ t(3), round(0.005 * cols) columns x100."""
    A = student_t3((rows, cols), seed=20, device=device)
    outlier_columns(A, max(1, round(0.005 * cols)), 100.0, seed=20)
    return {"A": to_bf16(A)}


def llama8b_up(device="cpu", T: int = 8192, K: int = 4096, N: int = 14336):
    X = student_t3((T, K), seed=30, device=device)
    W = normal((N, K), 0.02, seed=31, device=device)
    dY = normal((T, N), 1e-3, seed=32, device=device)
    rho = student_t3((T, 1), seed=33, device=device).abs()
    dY *= rho
    return {"X": to_bf16(X), "W": to_bf16(W), "dY": to_bf16(dY)}


def blocks_2d(device="cpu", T: int = 8192, K: int = 4096, N: int = 14336):
    W = student_t3((N, K), seed=40, device=device)
    outlier_columns(W, max(1, round(0.005 * K)), 100.0, seed=40)
    dY = student_t3((T, N), seed=41, device=device)
    outlier_columns(dY, max(1, round(0.005 * N)), 100.0, seed=41)
    X = student_t3((T, K), seed=42, device=device)
    return {"X": to_bf16(X), "W": to_bf16(W), "dY": to_bf16(dY)}


def llama70b_down(device="cpu", T: int = 16384, D: int = 8192, F: int = 28672):
    H = student_t3((T, F), seed=50, device=device)
    W = normal((D, F), 0.01, seed=51, device=device)
    dY = normal((T, D), 1e-3, seed=52, device=device)
    return {"H": to_bf16(H), "W": to_bf16(W), "dY": to_bf16(dY)}


def llama70b_attn_q(device="cpu", T: int = 16384, D: int = 8192, N: int = 8192):
    """Attention query projection of the 70B model, one GPU's share: X [T][D] ~ t(3) (the
    normalised layer input), Wq [N][D] ~ N(0, 0.01), dY [T][N] ~ N(0, 1e-3). N = 1024 gives the
    key projection (8 key/value heads of 128)."""
    X = student_t3((T, D), seed=60, device=device)
    W = normal((N, D), 0.01, seed=61, device=device)
    dY = normal((T, N), 1e-3, seed=62, device=device)
    return {"X": to_bf16(X), "W": to_bf16(W), "dY": to_bf16(dY)}
