"""dsa_measure_peaks on the GPU: the attainable rates the bench reports next
to the spec-sheet peaks.  Each must be positive and below its spec-sheet
figure (bf16 2.5 PFLOP/s and FP8 5.0 PFLOP/s dense, HBM 8 TB/s) with some
margin for clock boosts, and the loops must run at more than a small fraction
of it (a loop that measured launch overhead or a compiler-removed body would
not)."""
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_16_amd as m  # fails loudly when libdsa.so is missing
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return m


def test_measure_peaks(dsa):
    say("[peaks] MFMA loops, streaming read and copy over 512 MiB")
    buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    p = dsa.measure_peaks(buf)
    say(f"  {p}")
    for key, spec in (("bf16_tflops", 2500.0), ("fp8_tflops", 5000.0), ("hbm_read_gbs", 8000.0),
                      ("hbm_copy_gbs", 8000.0)):
        assert 0.1 * spec < p[key] < 1.1 * spec, (key, p[key])
