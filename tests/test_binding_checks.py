"""CPU checks of the Python binding's argument validation: caller-supplied buffers are checked
(device, dtype, exact shape, contiguity) before their addresses reach a kernel, and the linear
op's configuration refuses option sets that one shared tile quantization cannot serve. Nothing
here launches GPU work or loads the HIP library."""
import pytest
import torch


@pytest.fixture(scope="module")
def mx(monkeypatch_module):
    import mxfp4_block_scaled_hadamard32_amd as m

    def no_library(*a, **k):
        raise AssertionError("the library was reached before the arguments were checked")
    monkeypatch_module.setattr(m, "lib", no_library)
    return m


@pytest.fixture(scope="module")
def monkeypatch_module():
    mp = pytest.MonkeyPatch()
    yield mp
    mp.undo()


CPU = torch.device("cpu")
U8 = (torch.uint8,)


def test_buf_accepts_a_matching_buffer(mx):
    t = torch.zeros((4, 8), dtype=torch.uint8)
    assert mx._buf(t, "codes", (4, 8), U8, CPU) is t


@pytest.mark.parametrize("bad, exc", [
    (torch.zeros((4, 9), dtype=torch.uint8), ValueError),          # undersized / wrong shape
    (torch.zeros((4, 8), dtype=torch.int8), TypeError),            # wrong dtype
    (torch.zeros((8, 4), dtype=torch.uint8).t(), ValueError),      # transposed view
    (torch.zeros((4, 16), dtype=torch.uint8)[:, :8], ValueError),  # strided slice
    (None, TypeError),
    (b"\x00" * 32, TypeError),
])
def test_buf_rejects_mismatches(mx, bad, exc):
    with pytest.raises(exc):
        mx._buf(bad, "codes", (4, 8), U8, CPU)


def test_buf_rejects_another_device(mx):
    t = torch.zeros((4, 8), dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError):
        mx._buf(t, "codes", (4, 8), U8, CPU)


def test_output_with_leading_dimension(mx):
    big = torch.zeros((4, 16), dtype=torch.float32)
    assert mx._buf(big[:, :8], "out", (4, 8), (torch.float32,), CPU, rows_only=True) is not None
    with pytest.raises(ValueError):  # columns not contiguous
        mx._buf(big[:, ::2], "out", (4, 8), (torch.float32,), CPU, rows_only=True)
    with pytest.raises(ValueError):  # wrong row count
        mx._buf(big[:3, :8], "out", (4, 8), (torch.float32,), CPU, rows_only=True)


def test_host_tensors_never_reach_the_library(mx):
    x = torch.zeros((32, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mx.mx_quantize(x)
    with pytest.raises(ValueError):
        mx.mx_quantize_2d(x)
    with pytest.raises(ValueError):
        mx.mx_scale_mismatch_map(x)
    q = torch.zeros((32, 32), dtype=torch.uint8)
    s = torch.zeros((32, 2), dtype=torch.uint8)
    with pytest.raises(ValueError):
        mx.mx_gemm_fprop(q, s, 1, q, s, 1)
    with pytest.raises(ValueError):
        mx.mx_gemm_mxfp8(q, s, 0, q, s, 0)
    with pytest.raises(ValueError):
        mx.mx_dequantize(q, s, 32, 64)


def test_linear_config_refuses_differing_specs_on_a_shared_tile():
    from mxfp4_block_scaled_hadamard32_amd import linear as lin
    sr = lin.QuantSpec(scale_rule=1, round=1)
    rne = lin.QuantSpec(scale_rule=1, round=0)
    # W tiles serve Fprop and Dgrad; dY tiles serve Dgrad and Wgrad
    for cfg in (lin.MXLinearConfig(w_block=32, fprop_q=rne, dgrad_q=sr, wgrad_q=sr),
                lin.MXLinearConfig(dy_block=64, fprop_q=rne, dgrad_q=sr, wgrad_q=rne),
                lin.MXLinearConfig(w_block=32, dy_block=32, fprop_q=sr, dgrad_q=sr,
                                   wgrad_q=lin.QuantSpec(scale_rule=0, round=1))):
        with pytest.raises(ValueError):
            cfg.check()
    # with one of the two GEMMs off the tile follows the other one's options
    cfg = lin.MXLinearConfig(w_block=32, fprop=False, fprop_q=rne, dgrad_q=sr)
    cfg.check()
    assert cfg.w_tile_spec() is sr
    cfg = lin.MXLinearConfig(dy_block=32, dgrad=False, dgrad_q=rne, wgrad_q=sr)
    cfg.check()
    assert cfg.dy_tile_spec() is sr
    # agreeing options (the sign mask plays no part in a tile) pass
    lin.MXLinearConfig(w_block=32, dy_block=32, fprop_q=sr, dgrad_q=sr,
                       wgrad_q=lin.QuantSpec(scale_rule=1, round=1, sign_mask=5)).check()
