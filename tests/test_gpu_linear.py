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
