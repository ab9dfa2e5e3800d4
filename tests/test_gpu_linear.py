"""The MXFP4 linear layer (forward and straight-through backward) against the oracle.

Each product is checked like the GEMM entry points: the oracle quantizes the same operands
along the same axes with the same options and seeds, forms the exact product in float64, and
the bf16 output must lie in the rounding bracket of the GEMM bound. A toggled-off product is
the bf16 reference product itself. A short synthetic regression trained through the layer
must reduce its loss.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.parity import check_gemm

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def lin():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_block_scaled_hadamard32_amd as m
    m.lib()
    from mxfp4_block_scaled_hadamard32_amd import linear
    return linear


def oracle_product(orc, a, a_axis, b, b_axis, spec, seed_a, seed_b, M, N, K):
    """2^alpha * A . B^T with A, B the oracle quantizations of a, b along the reduction axis."""
    aq, as_ = orc.quantize(wl.host_input(a), axis=a_axis, scale_rule=spec.scale_rule,
                           round_mode=spec.round, hadamard=spec.hadamard,
                           sign_mask=spec.sign_mask, seed=seed_a)
    bq, bs = orc.quantize(wl.host_input(b), axis=b_axis, scale_rule=spec.scale_rule,
                          round_mode=spec.round, hadamard=spec.hadamard,
                          sign_mask=spec.sign_mask, seed=seed_b)
    return orc.gemm(aq, as_, 1, bq, bs, 1, M, N, K, -5 if spec.hadamard else 0)


@pytest.mark.parametrize("variant", ["plain", "hadamard_sr"])
def test_linear_forward_backward_against_oracle(lin, orc, variant):
    T, K, N = 256, 512, 384
    if variant == "plain":
        spec = lin.QuantSpec()
        cfg = lin.MXLinearConfig(fprop_q=spec, dgrad_q=spec, wgrad_q=spec, seed=100)
    else:
        f = lin.QuantSpec(scale_rule=1, round=1, hadamard=1, sign_mask=0x9E3779B9)
        wq = lin.QuantSpec(scale_rule=1, round=0, hadamard=1, sign_mask=0)  # deterministic H
        cfg = lin.MXLinearConfig(fprop_q=f, dgrad_q=f, wgrad_q=wq, seed=100)
    x = wl.student_t3((T, K), seed=1).to(torch.bfloat16).to(DEV).requires_grad_(True)
    w = wl.normal((N, K), 0.05, seed=2).to(torch.bfloat16).to(DEV).requires_grad_(True)
    dy = wl.normal((T, N), 1e-3, seed=3).to(torch.bfloat16).to(DEV)
    y = lin.MXLinearFunction.apply(x, w, cfg)
    y.backward(dy)
    torch.cuda.synchronize()
    sx, sw, sdy = 100, 101, 102
    C, Cabs = oracle_product(orc, x.detach(), 1, w.detach(), 1, cfg.fprop_q, sx, sw, T, N, K)
    check_gemm(y.detach(), C, Cabs)
    C, Cabs = oracle_product(orc, dy, 1, w.detach(), 0, cfg.dgrad_q, sdy, sw, T, K, N)
    check_gemm(x.grad, C, Cabs)
    C, Cabs = oracle_product(orc, dy, 0, x.detach(), 0, cfg.wgrad_q, sdy, sx, N, K, T)
    check_gemm(w.grad, C, Cabs)


def test_linear_toggles_off_is_bf16(lin):
    T, K, N = 64, 128, 96
    cfg = lin.MXLinearConfig(fprop=False, dgrad=False, wgrad=False)
    x = torch.randn(T, K, device=DEV, dtype=torch.bfloat16, requires_grad=True)
    w = torch.randn(N, K, device=DEV, dtype=torch.bfloat16, requires_grad=True)
    dy = torch.randn(T, N, device=DEV, dtype=torch.bfloat16)
    y = lin.MXLinearFunction.apply(x, w, cfg)
    y.backward(dy)
    assert torch.equal(y, x.detach() @ w.detach().t())
    assert torch.equal(x.grad, dy @ w.detach())
    assert torch.equal(w.grad, dy.t() @ x.detach())


def test_linear_trains_synthetic_regression(lin):
    """Fit y* = x W*^T with every product in MXFP4 (Hadamard + SR on Fprop/Dgrad, deterministic
    Hadamard on Wgrad): the mean squared error must fall well below its starting value."""
    torch.manual_seed(0)
    T, K, N = 512, 256, 128
    f = lin.QuantSpec(scale_rule=1, round=1, hadamard=1, sign_mask=0x2545F491)
    wq = lin.QuantSpec(scale_rule=1, round=0, hadamard=1, sign_mask=0)
    layer = lin.MXLinear(K, N, lin.MXLinearConfig(fprop_q=f, dgrad_q=f, wgrad_q=wq))
    w_star = torch.randn(N, K, device=DEV) * K ** -0.5
    # the expected gradient of the mean over T x N outputs is (2/N)(W - W*): lr = N/8 takes a
    # quarter of the way to W* per step
    opt = torch.optim.SGD(layer.parameters(), lr=N / 8)
    losses = []
    for step in range(60):
        x = torch.randn(T, K, device=DEV)
        target = x @ w_star.t()
        y = layer(x.to(torch.bfloat16)).float()
        loss = ((y - target) ** 2).mean()
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(loss.item())
    assert np.isfinite(losses).all()
    assert np.mean(losses[-5:]) < 0.05 * losses[0], losses[::10]


def oracle_tiles(orc, t, B, spec, seed):
    """Oracle BxB tiles with the scales in the GEMM's layout (g = B, one byte per 32 k)."""
    c, s, ct, st = orc.quantize_2d_block(wl.host_input(t), B, scale_rule=spec.scale_rule,
                                         round_mode=spec.round, seed=seed)
    rep = B // 32
    return c, np.repeat(s, rep, axis=1), ct, np.repeat(st, rep, axis=1)


@pytest.mark.parametrize("w_block,dy_block", [(32, 32), (64, 1), (1, 64)])
def test_linear_tiled_operands_against_oracle(lin, orc, w_block, dy_block):
    """W and / or dY in square tiles: Fprop reads W's tiles, Dgrad their transposed copy, Dgrad
    and Wgrad dY's tiles and their transposed copy; X stays 1x32."""
    T, K, N = 256, 512, 384
    q = lin.QuantSpec(scale_rule=1, round=1)
    cfg = lin.MXLinearConfig(fprop_q=q, dgrad_q=q, wgrad_q=q, w_block=w_block, dy_block=dy_block,
                             seed=300)
    x = wl.student_t3((T, K), seed=11).to(torch.bfloat16).to(DEV).requires_grad_(True)
    w = wl.normal((N, K), 0.05, seed=12).to(torch.bfloat16).to(DEV).requires_grad_(True)
    dy = wl.normal((T, N), 1e-3, seed=13).to(torch.bfloat16).to(DEV)
    y = lin.MXLinearFunction.apply(x, w, cfg)
    y.backward(dy)
    torch.cuda.synchronize()
    sx, sw, sdy = 300, 301, 302
    hx = wl.host_input(x.detach())
    xq, xs = orc.quantize(hx, axis=1, scale_rule=1, round_mode=1, seed=sx)
    xtq, xts = orc.quantize(hx, axis=0, scale_rule=1, round_mode=1, seed=sx)
    if w_block > 1:
        wq, ws, wtq, wts = oracle_tiles(orc, w.detach(), w_block, q, sw)
    else:
        wq, ws = orc.quantize(wl.host_input(w.detach()), axis=1, scale_rule=1, round_mode=1, seed=sw)
        wtq, wts = orc.quantize(wl.host_input(w.detach()), axis=0, scale_rule=1, round_mode=1, seed=sw)
    if dy_block > 1:
        dyq, dys, dytq, dyts = oracle_tiles(orc, dy, dy_block, q, sdy)
    else:
        dyq, dys = orc.quantize(wl.host_input(dy), axis=1, scale_rule=1, round_mode=1, seed=sdy)
        dytq, dyts = orc.quantize(wl.host_input(dy), axis=0, scale_rule=1, round_mode=1, seed=sdy)
    C, Cabs = orc.gemm(xq, xs, 1, wq, ws, w_block, T, N, K)
    check_gemm(y.detach(), C, Cabs)
    C, Cabs = orc.gemm(dyq, dys, dy_block, wtq, wts, w_block, T, K, N)
    check_gemm(x.grad, C, Cabs)
    C, Cabs = orc.gemm(dytq, dyts, dy_block, xtq, xts, 1, N, K, T)
    check_gemm(w.grad, C, Cabs)


def test_linear_mxfp8_against_oracle(lin, orc):
    """fmt = "mxfp8": X and W in E4M3, dY in E5M2, every GEMM within the MXFP8 bound."""
    T, K, N = 256, 512, 384
    q = lin.QuantSpec(scale_rule=1, round=0)
    cfg = lin.MXLinearConfig(fprop_q=q, dgrad_q=q, wgrad_q=q, fmt="mxfp8", seed=500)
    x = wl.student_t3((T, K), seed=21).to(torch.bfloat16).to(DEV).requires_grad_(True)
    w = wl.normal((N, K), 0.05, seed=22).to(torch.bfloat16).to(DEV).requires_grad_(True)
    dy = wl.normal((T, N), 1e-3, seed=23).to(torch.bfloat16).to(DEV)
    y = lin.MXLinearFunction.apply(x, w, cfg)
    y.backward(dy)
    torch.cuda.synchronize()
    hx, hw, hdy = (wl.host_input(t.detach()) for t in (x, w, dy))
    rel = 2.0 ** -10  # the MXFP8 matrix-core bound
    f = dict(scale_rule=1)
    xq, xs = orc.quantize_fp8(hx, fmt=0, axis=1, **f)
    wq, ws = orc.quantize_fp8(hw, fmt=0, axis=1, **f)
    C, Cabs = orc.gemm_fp8(xq, xs, 0, wq, ws, 0, T, N, K)
    check_gemm(y.detach(), C, Cabs, rel=rel)
    dyq, dys = orc.quantize_fp8(hdy, fmt=1, axis=1, **f)
    wtq, wts = orc.quantize_fp8(hw, fmt=0, axis=0, **f)
    C, Cabs = orc.gemm_fp8(dyq, dys, 1, wtq, wts, 0, T, K, N)
    check_gemm(x.grad, C, Cabs, rel=rel)
    dytq, dyts = orc.quantize_fp8(hdy, fmt=1, axis=0, **f)
    xtq, xts = orc.quantize_fp8(hx, fmt=0, axis=0, **f)
    C, Cabs = orc.gemm_fp8(dytq, dyts, 1, xtq, xts, 0, N, K, T)
    check_gemm(w.grad, C, Cabs, rel=rel)


def test_linear_config_rejects_undefined_combinations(lin):
    x = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    for cfg in (lin.MXLinearConfig(w_block=16), lin.MXLinearConfig(fmt="fp6"),
                lin.MXLinearConfig(fmt="mxfp8", w_block=32),
                lin.MXLinearConfig(w_block=32, fprop_q=lin.QuantSpec(hadamard=1))):
        with pytest.raises(ValueError):
            lin.MXLinearFunction.apply(x, w, cfg)


def test_linear_trains_with_transposition_invariant_tiles(lin):
    """The 2-D recipe (W and dY in 32x32 tiles, X 1x32, ceil scale, SR): the synthetic
    regression of the MXFP4 test must also converge."""
    torch.manual_seed(1)
    T, K, N = 512, 256, 128
    q = lin.QuantSpec(scale_rule=1, round=1)
    layer = lin.MXLinear(K, N, lin.MXLinearConfig(fprop_q=q, dgrad_q=q, wgrad_q=q, w_block=32,
                                                  dy_block=32))
    w_star = torch.randn(N, K, device=DEV) * K ** -0.5
    opt = torch.optim.SGD(layer.parameters(), lr=N / 8)
    losses = []
    for _ in range(60):
        x = torch.randn(T, K, device=DEV)
        loss = ((layer(x.to(torch.bfloat16)).float() - x @ w_star.t()) ** 2).mean()
        opt.zero_grad()
        loss.backward()
        opt.step()
        losses.append(loss.item())
    assert np.isfinite(losses).all()
    assert np.mean(losses[-5:]) < 0.05 * losses[0], losses[::10]
