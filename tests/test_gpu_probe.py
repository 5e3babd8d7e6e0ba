"""GPU: the machine-rate probes (include/moe_probe.h) run and report rates
between a sane floor and the published MI355X peaks (HBM 8 TB/s; dense MFMA
2516.6 TFLOP/s bf16, 5033 TFLOP/s FP8).  The rates themselves are what the
harness reports; the bounds only catch a probe that is broken (a rate above
the peak means it did less work than it counts)."""
import pytest
import torch

import sparse_moe_layer_bias_amd as moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the probe tests need the HIP library on an MI355X")
    moe.lib()
    yield
    torch.cuda.synchronize()


def test_probe_hbm_read_rate():
    from sparse_moe_layer_bias_amd import probe
    r = probe.hbm_read_rate(nbytes=1 << 30, blocks=512, reps=3)
    print("hbm read %.0f GB/s" % (r / 1e9), flush=True)
    assert 1.0e12 < r < 8.0e12 * 1.02


@pytest.mark.parametrize("dtype,peak", [("bf16", 2516.6e12), ("fp8", 5033e12)])
def test_probe_mfma_rate(dtype, peak):
    from sparse_moe_layer_bias_amd import probe
    r = probe.mfma_rate(dtype, iters=1000, blocks=256, reps=2)
    print("%s MFMA %.0f TFLOP/s" % (dtype, r / 1e12), flush=True)
    assert 0.2 * peak < r < 1.02 * peak
