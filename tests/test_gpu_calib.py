"""The matrix-core rate measurement (rvq_mfma_rate): a rate and a clock in
the range the chip can hold, and zero operands no slower than random ones."""
import pytest
import torch

pytestmark = pytest.mark.gpu

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 at the nominal 2.4 GHz


@pytest.fixture(scope="module")
def rvq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import residual_vector_quantization_rvq_amd as m
    return m


def test_rate_and_clock_in_range(rvq):
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rnd, ghz_r = rvq.rvq_mfma_rate(cus, 20_000, False, dev)
    zero, ghz_z = rvq.rvq_mfma_rate(cus, 20_000, True, dev)
    print(f"random {rnd:.1f} TFLOP/s at {ghz_r:.3f} GHz, zero {zero:.1f} TFLOP/s at {ghz_z:.3f} GHz")
    for tf, ghz in ((rnd, ghz_r), (zero, ghz_z)):
        assert 0.05 * PEAK_BF16_TFLOPS < tf <= 1.02 * PEAK_BF16_TFLOPS
        assert 0.3 < ghz < 2.6
        # one MFMA of 32 cycles per SIMD at most: the rate cannot exceed the
        # clock's share of the nominal peak
        assert tf <= PEAK_BF16_TFLOPS * ghz / 2.4 * 1.05
    assert zero >= 0.98 * rnd
