"""Helpers shared by the GPU parity tests (comparison rules; no method arithmetic)."""
import numpy as np
import torch

GEMM_REL = 2.0 ** -20  # |gpu - exact| <= 2^-20 * sum_k |a_k b_k|, fp32 accumulation


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """Exact round-to-nearest-even of float64 values to bfloat16 (8 significant bits), returned as
    float64. Overflow goes to +-inf."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    finite = np.isfinite(x)
    out[~finite] = x[~finite]
    xf = x[finite]
    m, e = np.frexp(xf)  # xf = m * 2^e, |m| in [0.5, 1)
    # quantum 2^(e-8) for normal bf16, at least 2^-133 (bf16 subnormal step)
    qexp = np.maximum(e - 8, -133)
    q = np.ldexp(1.0, qexp)
    r = np.rint(xf / q) * q  # np.rint: round half to even, exact here
    big = np.abs(r) > 3.3895313892515355e38  # beyond the largest finite bf16
    r[big] = np.copysign(np.inf, r[big])
    out[finite] = r
    return out


def check_gemm(gpu: torch.Tensor, C: np.ndarray, Cabs: np.ndarray, rows=None, cols=None,
               rel: float = GEMM_REL):
    """fp32 output: elementwise |gpu - C| <= rel * Cabs (rel = 2^-20 by default). bf16 output:
    the rounding of any value within that bound, i.e. RNE(C - b) <= gpu <= RNE(C + b) (rounding
    is monotone)."""
    g = gpu
    if rows is not None:
        g = g[torch.as_tensor(rows, device=g.device)]
    if cols is not None:
        g = g[:, torch.as_tensor(cols, device=g.device)]
    got = g.float().cpu().numpy().astype(np.float64)
    bound = rel * Cabs
    if gpu.dtype == torch.float32:
        err = np.abs(got - C)
        bad = ~(err <= bound)
        assert not bad.any(), (f"{bad.sum()} of {bad.size} outside bound; worst excess "
                               f"{np.max(err - bound)} at {np.argwhere(bad)[:5].tolist()}")
    else:
        lo = bf16_round_f64(C - bound)
        hi = bf16_round_f64(C + bound)
        bad = ~((got >= lo) & (got <= hi))
        assert not bad.any(), (f"{bad.sum()} of {bad.size} outside bf16 bracket, e.g. "
                               f"{[(got[tuple(i)], C[tuple(i)]) for i in np.argwhere(bad)[:3]]}")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def assert_bytes_equal(gpu: torch.Tensor, ref: np.ndarray, what: str, rows=None):
    got = host(gpu)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    if not np.array_equal(got, ref):
        diff = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(diff)} of {got.size} bytes differ; first at "
                             f"{diff[:4].tolist()} gpu={got[tuple(diff[0])]:#04x} "
                             f"oracle={ref[tuple(diff[0])]:#04x}")
