"""Fprop with the output quantized in the GEMM epilogue (mx_gemm_fprop_quant), against the oracle.

The kernel quantizes its own fp32 accumulator values. Their accumulation order is not fixed by
the method, and any fp32 result within the GEMM bound |y - C| <= 2^-20 sum|a b| is a correct
product, so the check is: every scale byte and every code is the quantization of some fp32
output within that bound, computed by the oracle. The scale is monotone in the block maximum
and, for a fixed random field, the rounding is monotone in the value, so it suffices to bracket
each block's maximum and each element between the oracle's results at the interval ends. With
the Hadamard rotation the interval is carried through the transform (the sum of the 32 input
half-widths plus the fp32 error bound of five butterfly stages, 6 * 2^-24 * sum|x|). Almost all
codes are unique under that interval, and the test also requires that.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.parity import host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GEMM_REL = 2.0 ** -20


@pytest.fixture(scope="module")
def mx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_block_scaled_hadamard32_amd as m
    m.lib()
    return m


def hadamard_matrix(orc):
    """H32 as the oracle's transform applied to the unit vectors (entries are exactly +-1)."""
    eye = np.eye(32, dtype=np.float32)
    return np.stack([orc.fwht32(eye[j]) for j in range(32)], axis=1).astype(np.float64)


def outward_f32(lo, hi):
    lo32 = lo.astype(np.float32)
    hi32 = hi.astype(np.float32)
    lo32 = np.where(lo32.astype(np.float64) > lo, np.nextafter(lo32, np.float32(-np.inf)), lo32)
    hi32 = np.where(hi32.astype(np.float64) < hi, np.nextafter(hi32, np.float32(np.inf)), hi32)
    return lo32, hi32


def check_epilogue_quant(orc, codes, scales, C, Cabs, had, mask, rule, rnd, seed, rows=None):
    """C, Cabs: the oracle's product on all rows, or on the output rows `rows` (then codes and
    scales are the kernel's full outputs and are sliced to those rows)."""
    T, N = C.shape
    if rows is not None:
        sel = torch.as_tensor(rows, device=codes.device)
        codes, scales = codes[sel], scales[sel]
    row_of = np.arange(T) if rows is None else np.asarray(rows)
    nb = N // 32
    bound = GEMM_REL * Cabs
    Cb = C.reshape(T, nb, 32)
    Bb = bound.reshape(T, nb, 32)
    if had:
        H = hadamard_matrix(orc)
        D = np.array([-1.0 if (mask >> j) & 1 else 1.0 for j in range(32)])
        y = (Cb * D) @ H.T
        hw = Bb.sum(-1, keepdims=True) + 6 * 2.0 ** -24 * (np.abs(Cb) + Bb).sum(-1, keepdims=True)
        hw = np.broadcast_to(hw, y.shape)
    else:
        y, hw = Cb, Bb
    lo, hi = y - hw, y + hw
    # block maximum bracket -> scale byte bracket
    amin = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi))).max(-1)
    amax = np.maximum(np.abs(lo), np.abs(hi)).max(-1)
    amin32, _ = outward_f32(amin, amin)
    _, amax32 = outward_f32(amax, amax)
    sc = host(scales).astype(np.int64).reshape(T, nb)
    for t in range(T):
        for b in range(nb):
            e_lo = orc.scale_exponent(float(amin32[t, b]), rule) + 127
            e_hi = orc.scale_exponent(float(amax32[t, b]), rule) + 127
            assert e_lo <= sc[t, b] <= e_hi, (t, b, sc[t, b], e_lo, e_hi)
    # codes, with the scale the kernel chose
    cd = host(codes).reshape(T, N // 2)
    got = np.empty((T, N), dtype=np.int64)
    got[:, 0::2] = cd & 0xF
    got[:, 1::2] = cd >> 4
    e = (sc - 127).astype(np.float64)
    f = np.repeat(2.0 ** -e, 32, axis=1)
    vlo, vhi = outward_f32(lo.reshape(T, N) * f, hi.reshape(T, N) * f)
    unique = 0
    for t in range(T):
        for n in range(N):
            r = orc.sr_field(seed, int(row_of[t]) * N + n) if rnd else 0
            c_lo = orc.e2m1_encode(float(vlo[t, n]), rnd, r)
            c_hi = orc.e2m1_encode(float(vhi[t, n]), rnd, r)
            d = orc.e2m1_decode(int(got[t, n]))
            assert orc.e2m1_decode(c_lo) <= d <= orc.e2m1_decode(c_hi), \
                (t, n, int(got[t, n]), c_lo, c_hi, float(vlo[t, n]), float(vhi[t, n]))
            unique += c_lo == c_hi
    assert unique >= 0.97 * T * N, f"only {unique} of {T * N} codes are fixed by the bound"


def operands(mx, T, N, K, seed):
    x = wl.student_t3((T, K), seed=seed).to(torch.bfloat16).to(DEV)
    w = wl.normal((N, K), 0.05, seed=seed + 1).to(torch.bfloat16).to(DEV)
    xq, xs = mx.mx_quantize(x, scale_rule=1)
    wq, ws = mx.mx_quantize(w, scale_rule=1)
    return xq, xs, wq, ws


@pytest.mark.parametrize("T,N,K", [(288, 320, 1024),   # partial row and column tiles, 256-k steps
                                   (256, 96, 384)])    # 128-k steps
@pytest.mark.parametrize("rule,rnd,had,mask", [(0, 0, 0, 0), (1, 1, 1, 0x9E3779B9),
                                               (1, 0, 1, 0), (0, 1, 0, 0)])
def test_fprop_quant_epilogue(mx, orc, T, N, K, rule, rnd, had, mask):
    xq, xs, wq, ws = operands(mx, T, N, K, seed=T + N + K)
    alpha = -3
    codes, scales = mx.mx_gemm_fprop_quant(xq, xs, 1, wq, ws, 1, alpha_exp=alpha, scale_rule=rule,
                                           round=rnd, hadamard=had, sign_mask=mask, seed=77)
    torch.cuda.synchronize()
    C, Cabs = orc.gemm(host(xq), host(xs), 1, host(wq), host(ws), 1, T, N, K, alpha)
    check_epilogue_quant(orc, codes, scales, C, Cabs, had, mask, rule, rnd, 77)


@pytest.mark.parametrize("K", [512, 1024])
def test_fprop_quant_matches_separate_quantize_where_exact(mx, orc, K):
    """Small integers times power-of-two scales make every fp32 accumulation exact, so the fused
    output must equal mx_quantize of mx_gemm_fprop's fp32 output byte for byte (both kernels:
    128-k steps, and 256-k steps with two waves per SIMD)."""
    T, N = 64, 256
    g = torch.Generator().manual_seed(5)
    x = torch.randint(-6, 7, (T, K), generator=g).float()
    w = torch.randint(-6, 7, (N, K), generator=g).float() * 0.5
    xq, xs = mx.mx_quantize(x.to(DEV), scale_rule=1)
    wq, ws = mx.mx_quantize(w.to(DEV), scale_rule=1)
    y = mx.mx_gemm_fprop(xq, xs, 1, wq, ws, 1, out_dtype=torch.float32)
    for rule, rnd, had, mask in [(0, 0, 0, 0), (1, 1, 1, 0x12345678)]:
        c1, s1 = mx.mx_gemm_fprop_quant(xq, xs, 1, wq, ws, 1, scale_rule=rule, round=rnd,
                                        hadamard=had, sign_mask=mask, seed=9)
        c2, s2 = mx.mx_quantize(y, scale_rule=rule, round=rnd, hadamard=had, sign_mask=mask,
                                seed=9)
        assert torch.equal(s1, s2) and torch.equal(c1, c2)


def test_fprop_quant_chained_tiles(mx, orc):
    """More output tiles than compute units (each workgroup walks several), partial edge tiles,
    Hadamard with random signs, ceil scale and stochastic rounding in the epilogue."""
    T, N, K = 4352, 4128, 1024
    xq, xs, wq, ws = operands(mx, T, N, K, seed=3)
    codes, scales = mx.mx_gemm_fprop_quant(xq, xs, 1, wq, ws, 1, alpha_exp=-5, scale_rule=1,
                                           round=1, hadamard=1, sign_mask=0x9E3779B9, seed=5)
    torch.cuda.synchronize()
    rows = np.array([0, 255, 256, 2049, 4100, T - 1])
    C, Cabs = orc.gemm(host(xq), host(xs), 1, host(wq), host(ws), 1, T, N, K, -5, rows=rows)
    check_epilogue_quant(orc, codes, scales, C, Cabs, 1, 0x9E3779B9, 1, 1, 5, rows=rows)


def test_fprop_quant_rejects_ragged_k(mx):
    xq = torch.zeros((32, 48), dtype=torch.uint8, device=DEV)   # K = 96
    xs = torch.zeros((32, 3), dtype=torch.uint8, device=DEV)
    with pytest.raises(mx.MxError):
        mx.mx_gemm_fprop_quant(xq, xs, 1, xq, xs, 1)
