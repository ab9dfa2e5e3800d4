"""The matrix-core ceiling probe (libmx_probe.so) runs and reports a rate below the dense FP4
peak; bench.py prices the GEMMs against it as well as against the peak."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_mfma_probe_rate_is_plausible():
    import bench
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    rate = bench.mfma_ceiling(torch, workgroups=512, iters=200, reps=2)
    assert 1000.0 < rate < bench.PEAK_FP4_TFLOPS * 1.02, rate
