"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Every kernel runs on the full tensors; the oracle checks them where it can in seconds:
the tiny and quantize-stream workloads in full, the large ones on sampled row blocks (codes and
scales bit-exact) and on sampled GEMM outputs (within 2^-20 * sum|ab| or its bf16 bracket).
"""
import os

import numpy as np
import pytest
import torch

import workloads as wl
from tests.parity import assert_bytes_equal, check_gemm, host

pytestmark = pytest.mark.gpu

DEV = "cuda"
THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_hadamard32_amd as m
    assert torch.cuda.is_available()
    m.lib()
    return m


def row_samples(rows, count=2, block=64, seed=0):
    """A few aligned row ranges: the first, the last and random ones in between."""
    rng = np.random.default_rng(seed)
    starts = {0, rows - block}
    while len(starts) < count + 2:
        starts.add(int(rng.integers(0, rows // block)) * block)
    return sorted((s, s + block) for s in starts)


def check_quant_rows(orc, x_dev, codes, scales, axis, ranges, **opts):
    """Compare the GPU outputs of a full-tensor quantize with the oracle on row ranges."""
    x = wl.host_input(x_dev)
    for r0, r1 in ranges:
        rc, rs = orc.quantize(x, axis=axis, row_range=(r0, r1), nthreads=THREADS, **opts)
        if axis == 1:
            assert_bytes_equal(scales[r0:r1], rs[r0:r1], f"scales rows {r0}:{r1}")
            assert_bytes_equal(codes[r0:r1], rc[r0:r1], f"codes rows {r0}:{r1}")
        else:
            assert_bytes_equal(scales[:, r0 // 32:r1 // 32], rs[:, r0 // 32:r1 // 32],
                               f"scales_t rows {r0}:{r1}")
            assert_bytes_equal(codes[:, r0 // 2:r1 // 2], rc[:, r0 // 2:r1 // 2],
                               f"codes_t rows {r0}:{r1}")


def check_gemm_sampled(orc, out, aq, as_, ga, bq, bs, gb, alpha, seed=0, nrows=6, ncols=768):
    M, N, K = aq.shape[0], bq.shape[0], 2 * aq.shape[1]
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, nrows)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, ncols)]))
    C, Cabs = orc.gemm(host(aq), host(as_), ga, host(bq), host(bs), gb, M, N, K, alpha,
                       rows=rows, cols=cols)
    check_gemm(out, C, Cabs, rows=rows, cols=cols)


# ------------------------------------------------------------------------------------------------
def test_tiny_full(mx, orc):
    """X, W 256x256 fp32, floor scale, RNE, no Hadamard; one 256^3 GEMM, fp32 out; all checked."""
    d = wl.tiny()
    X, W = d["X"].to(DEV), d["W"].to(DEV)
    xq, xs = mx.mx_quantize(X, scale_rule=0, round=0)
    wq, ws = mx.mx_quantize(W, scale_rule=0, round=0)
    y = mx.mx_gemm_fprop(xq, xs, 1, wq, ws, 1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rxq, rxs = orc.quantize(wl.host_input(d["X"]), scale_rule=0, round_mode=0)
    rwq, rws = orc.quantize(wl.host_input(d["W"]), scale_rule=0, round_mode=0)
    assert_bytes_equal(xs, rxs, "X scales")
    assert_bytes_equal(xq, rxq, "X codes")
    assert_bytes_equal(ws, rws, "W scales")
    assert_bytes_equal(wq, rwq, "W codes")
    C, Cabs = orc.gemm(rxq, rxs, 1, rwq, rws, 1, 256, 256, 256, 0)
    check_gemm(y, C, Cabs)


def test_quant_stream_full(mx, orc):
    """8192x4096 bf16, Hadamard with random signs, ceil scale, SR (seed 1234); every code and
    scale compared."""
    A = wl.quant_stream(device=DEV)["A"]
    mask = wl.sign_mask()
    c, s = mx.mx_quantize(A, scale_rule=1, round=1, hadamard=1, sign_mask=mask, seed=wl.SR_SEED)
    torch.cuda.synchronize()
    rc, rs = orc.quantize(wl.host_input(A), scale_rule=1, round_mode=1, hadamard=1,
                          sign_mask=mask, seed=wl.SR_SEED, nthreads=THREADS)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


# ------------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def llama8b(mx):
    d = wl.llama8b_up(device=DEV)
    X, W, dY = d["X"], d["W"], d["dY"]
    q = {}
    q["Xq"] = mx.mx_quantize(X, axis=1, scale_rule=0, round=0)
    q["Wq"] = mx.mx_quantize(W, axis=1, scale_rule=0, round=0)
    q["dYq"] = mx.mx_quantize(dY, axis=1, scale_rule=0, round=0)
    q["Wt"] = mx.mx_quantize(W, axis=0, scale_rule=0, round=0)
    q["dYt"] = mx.mx_quantize(dY, axis=0, scale_rule=0, round=0, hadamard=1, sign_mask=0)
    q["Xt"] = mx.mx_quantize(X, axis=0, scale_rule=0, round=0, hadamard=1, sign_mask=0)
    out = {
        "Y": mx.mx_gemm_fprop(*q["Xq"], 1, *q["Wq"], 1, alpha_exp=0),
        "dX": mx.mx_gemm_dgrad(*q["dYq"], 1, *q["Wt"], 1, alpha_exp=0),
        "dW": mx.mx_gemm_wgrad(*q["dYt"], 1, *q["Xt"], 1, alpha_exp=-5),
    }
    torch.cuda.synchronize()
    return d, q, out


@pytest.mark.parametrize("name,src,axis,had", [("Xq", "X", 1, 0), ("Wq", "W", 1, 0),
                                               ("dYq", "dY", 1, 0), ("Wt", "W", 0, 0),
                                               ("dYt", "dY", 0, 1), ("Xt", "X", 0, 1)])
def test_llama8b_quantize_sampled(orc, llama8b, name, src, axis, had):
    d, q, _ = llama8b
    x = d[src]
    check_quant_rows(orc, x, *q[name], axis, row_samples(x.shape[0], count=6, seed=len(name)),
                     scale_rule=0, round_mode=0, hadamard=had, sign_mask=0)


@pytest.mark.parametrize("gemm", ["fprop", "dgrad", "wgrad"])
def test_llama8b_gemm_sampled(orc, llama8b, gemm):
    _, q, out = llama8b
    a, b, o, alpha = {"fprop": ("Xq", "Wq", "Y", 0), "dgrad": ("dYq", "Wt", "dX", 0),
                      "wgrad": ("dYt", "Xt", "dW", -5)}[gemm]
    check_gemm_sampled(orc, out[o], *q[a], 1, *q[b], 1, alpha, seed=len(gemm))


def test_llama8b_wgrad_fp32_full_k(mx, orc, llama8b):
    """Wgrad's reduction runs over all T = 8192 tokens; with fp32 output the accumulated sum is
    held to 2^-20 * sum|ab| (no bf16 bracket to hide in) on 16 rows x 1024 columns."""
    _, q, _ = llama8b
    dW = mx.mx_gemm_wgrad(*q["dYt"], 1, *q["Xt"], 1, alpha_exp=-5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_gemm_sampled(orc, dW, *q["dYt"], 1, *q["Xt"], 1, -5, seed=11, nrows=16, ncols=1024)


# ------------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def blocks2d(mx):
    d = wl.blocks_2d(device=DEV)
    X, W, dY = d["X"], d["W"], d["dY"]
    q = {}
    q["W2"] = mx.mx_quantize_2d(W, scale_rule=1, round=0)                        # RTN on weights
    q["dY2"] = mx.mx_quantize_2d(dY, scale_rule=1, round=1, seed=wl.SR_SEED + 2)  # SR on gradients
    q["Xt"] = mx.mx_quantize(X, axis=0, scale_rule=1, round=0)                    # 1x32 along T
    Wc, Ws, Wct, Wst = q["W2"]
    dc, ds, dct, dst = q["dY2"]
    out = {
        # Dgrad dX = dY W: dY row-major 2-D codes, W's transposed 2-D codes (no re-quantization)
        "dX": mx.mx_gemm_dgrad(dc, ds, 32, Wct, Wst, 32),
        # Wgrad dW = dY^T X: dY's transposed 2-D codes, X along T
        "dW": mx.mx_gemm_wgrad(dct, dst, 32, *q["Xt"], 1),
    }
    torch.cuda.synchronize()
    return d, q, out


def test_blocks2d_transposition_invariance(mx, blocks2d):
    """scales(W) == scales(W^T)^T and the codes of W^T equal W's transposed copy."""
    d, q, _ = blocks2d
    Wt = d["W"].t().contiguous()
    c2, s2, ct2, st2 = mx.mx_quantize_2d(Wt, scale_rule=1, round=0)
    Wc, Ws, Wct, Wst = q["W2"]
    assert torch.equal(Ws, s2.t()) and torch.equal(Wst, s2)
    assert torch.equal(Wct, c2) and torch.equal(Wc, ct2)


@pytest.mark.parametrize("name,src,rnd,seed", [("W2", "W", 0, 0), ("dY2", "dY", 1, wl.SR_SEED + 2)])
def test_blocks2d_quantize_sampled(orc, blocks2d, name, src, rnd, seed):
    d, q, _ = blocks2d
    x = wl.host_input(d[src])
    c, s, ct, st = q[name]
    for r0, r1 in row_samples(x.shape[0], seed=rnd):
        rc, rs, rct, rst = orc.quantize_2d(x, scale_rule=1, round_mode=rnd, seed=seed,
                                           row_range=(r0, r1), nthreads=THREADS)
        assert_bytes_equal(s[r0 // 32:r1 // 32], rs[r0 // 32:r1 // 32], "scales")
        assert_bytes_equal(st[:, r0 // 32:r1 // 32], rst[:, r0 // 32:r1 // 32], "scales_t")
        assert_bytes_equal(c[r0:r1], rc[r0:r1], "codes")
        assert_bytes_equal(ct[:, r0 // 2:r1 // 2], rct[:, r0 // 2:r1 // 2], "codes_t")


def test_blocks2d_x_along_t_sampled(orc, blocks2d):
    d, q, _ = blocks2d
    check_quant_rows(orc, d["X"], *q["Xt"], 0, row_samples(d["X"].shape[0], seed=5),
                     scale_rule=1, round_mode=0)


@pytest.mark.parametrize("gemm", ["dgrad", "wgrad"])
def test_blocks2d_gemm_sampled(orc, blocks2d, gemm):
    _, q, out = blocks2d
    Wc, Ws, Wct, Wst = q["W2"]
    dc, ds, dct, dst = q["dY2"]
    if gemm == "dgrad":
        check_gemm_sampled(orc, out["dX"], dc, ds, 32, Wct, Wst, 32, 0, seed=3)
    else:
        check_gemm_sampled(orc, out["dW"], dct, dst, 32, *q["Xt"], 1, 0, seed=4)


# ------------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def llama70b(mx):
    """The benchmark's workload and launches (bench.Layer), run once."""
    import bench
    layer = bench.Layer(mx, wl, "llama70b_down")
    layer.step()
    torch.cuda.synchronize()
    return layer


@pytest.mark.parametrize("name,src,axis", [("Xq", "X", 1), ("Wq", "W", 1), ("dYq", "dY", 1),
                                           ("Wt", "W", 0), ("dYt", "dY", 0), ("Xt", "X", 0)])
def test_llama70b_quantize_sampled(orc, llama70b, name, src, axis):
    L = llama70b
    had, mask, rule, rnd = L.fprop_q
    x = getattr(L, src)
    check_quant_rows(orc, x, *L.buf[name], axis, row_samples(x.shape[0], count=3, seed=axis),
                     scale_rule=rule, round_mode=rnd, hadamard=had, sign_mask=mask,
                     seed=L.seeds[src])


@pytest.mark.parametrize("gemm", ["fprop", "dgrad", "wgrad"])
def test_llama70b_gemm_sampled(orc, llama70b, gemm):
    L = llama70b
    a, b, o = {"fprop": ("Xq", "Wq", L.Y), "dgrad": ("dYq", "Wt", L.dX),
               "wgrad": ("dYt", "Xt", L.dW)}[gemm]
    check_gemm_sampled(orc, o, *L.buf[a], 1, *L.buf[b], 1, L.alpha[gemm], seed=len(gemm),
                       nrows=4, ncols=512)


@pytest.mark.parametrize("gemm", ["fprop", "dgrad", "wgrad"])
def test_llama70b_gemm_fp32_full_k(mx, orc, llama70b, gemm):
    """The same operands with fp32 output, so the full-length sums (Fprop K = 28672, Dgrad
    K = 8192, Wgrad K = T = 16384) are held to 2^-20 * sum|ab| on 16 rows x 1024 columns."""
    L = llama70b
    a, b = {"fprop": ("Xq", "Wq"), "dgrad": ("dYq", "Wt"), "wgrad": ("dYt", "Xt")}[gemm]
    fn = getattr(mx, "mx_gemm_" + gemm)
    o = fn(*L.buf[a], 1, *L.buf[b], 1, alpha_exp=L.alpha[gemm], out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_gemm_sampled(orc, o, *L.buf[a], 1, *L.buf[b], 1, L.alpha[gemm], seed=7 + len(gemm),
                       nrows=16, ncols=1024)


@pytest.mark.parametrize("src", ["X", "dY"])
@pytest.mark.parametrize("rule", [1, 0])
def test_llama70b_columns_sr_without_transform_sampled(mx, orc, llama70b, src, rule):
    """Stochastic rounding without the transform down the columns (T) of the full-size 70B
    operands (H 16384x28672, dY 16384x8192): the column kernel's six-waves-per-SIMD variant."""
    L = llama70b
    x = getattr(L, src)
    c, s = mx.mx_quantize(x, axis=0, scale_rule=rule, round=1, hadamard=0, seed=4321)
    torch.cuda.synchronize()
    check_quant_rows(orc, x, c, s, 0, row_samples(x.shape[0], count=2, seed=11),
                     scale_rule=rule, round_mode=1, hadamard=0, seed=4321)
    del c, s


@pytest.mark.parametrize("fmt", [0, 1])
def test_mxfp8_columns_sr_without_transform_sampled(mx, orc, llama70b, fmt):
    """MXFP8 (E4M3, E5M2) with stochastic rounding and no transform down the columns of the
    full-size 16384x8192 dY: the MXFP8 column kernel's six-waves-per-SIMD variant, on sampled
    row ranges."""
    x = llama70b.dY
    c, s = mx.mx_quantize_mxfp8(x, fmt=fmt, axis=0, scale_rule=1, round=1, hadamard=0, seed=77)
    torch.cuda.synchronize()
    xh = wl.host_input(x)
    for r0, r1 in row_samples(x.shape[0], count=2, seed=12):
        rc, rs = orc.quantize_fp8(xh, fmt=fmt, axis=0, scale_rule=1, round_mode=1, hadamard=0,
                                  seed=77, row_range=(r0, r1))
        assert_bytes_equal(s[:, r0 // 32:r1 // 32], rs[:, r0 // 32:r1 // 32], f"scales_t {r0}:{r1}")
        assert_bytes_equal(c[:, r0:r1], rc[:, r0:r1], f"codes_t {r0}:{r1}")
    del c, s
