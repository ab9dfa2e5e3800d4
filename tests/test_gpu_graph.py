"""The layer step captured in a HIP graph.

No entry point allocates device memory or clears memory with a memset, so a whole step (six
operand quantizations and the three GEMMs) can be captured once and replayed. Each replay runs
on new inputs copied in eagerly between replays, and every replay must equal the eager step on
the same inputs bit for bit (same kernels, same launch configuration).
"""
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_hadamard32_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def test_step_replays_in_a_graph(mx):
    T, K, N = 512, 1024, 384
    mask = wl.sign_mask()
    X = torch.empty((T, K), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((N, K), dtype=torch.bfloat16, device=DEV)
    dY = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=DEV)  # noqa: E731
    buf = {"xq": (u8(T, K // 2), u8(T, K // 32)), "wq": (u8(N, K // 2), u8(N, K // 32)),
           "dyq": (u8(T, N // 2), u8(T, N // 32)), "wt": (u8(K, N // 2), u8(K, N // 32)),
           "dyt": (u8(N, T // 2), u8(N, T // 32)), "xt": (u8(K, T // 2), u8(K, T // 32))}
    Y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    dX = torch.empty((T, K), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((N, K), dtype=torch.float32, device=DEV)
    opts = dict(scale_rule=1, round=1, hadamard=1, sign_mask=mask)

    def step(stream):
        for name, src, axis, seed in (("xq", X, 1, 1), ("wq", W, 1, 2), ("dyq", dY, 1, 3),
                                      ("wt", W, 0, 2), ("dyt", dY, 0, 3), ("xt", X, 0, 1)):
            c, s = buf[name]
            mx.mx_quantize(src, axis=axis, seed=seed, codes=c, scales=s, stream=stream, **opts)
        mx.mx_gemm_fprop(*buf["xq"], 1, *buf["wq"], 1, alpha_exp=-5, out=Y, stream=stream)
        mx.mx_gemm_dgrad(*buf["dyq"], 1, *buf["wt"], 1, alpha_exp=-5, out=dX, stream=stream)
        mx.mx_gemm_wgrad(*buf["dyt"], 1, *buf["xt"], 1, alpha_exp=-5, out=dW, stream=stream)

    def fill(seed):
        X.copy_(wl.student_t3((T, K), seed=seed).to(torch.bfloat16))
        W.copy_(wl.normal((N, K), 0.02, seed=seed + 1).to(torch.bfloat16))
        dY.copy_(wl.normal((T, N), 1e-3, seed=seed + 2).to(torch.bfloat16))

    def outputs():
        return [t.clone() for t in (Y, dX, dW)] + [t.clone() for p in buf.values() for t in p]

    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()

    for rep, seed in enumerate((10, 20, 30)):
        fill(seed)
        torch.cuda.synchronize()
        step(None)  # eager reference on the same inputs
        torch.cuda.synchronize()
        eager = outputs()
        for t in (Y, dX, dW):
            t.fill_(float("nan"))
        for pair in buf.values():
            for t in pair:
                t.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outputs())):
            assert torch.equal(a, b), (rep, i)
        assert torch.isfinite(Y.float()).all() and torch.isfinite(dW).all()
