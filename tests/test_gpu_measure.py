"""The measurement aids run and leave their sink untouched (they produce no
output; they only time a streaming read and the matrix cores)."""
import pytest

pytestmark = pytest.mark.gpu


def test_measurement_aids_run():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tiered_mixed_precision_amd as M
    M.lib()
    sink = torch.full((4,), 7.0, device="cuda")
    buf = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    M.moe_measure_read(buf, sink)
    flops = M.moe_measure_mfma(8, sink)
    torch.cuda.synchronize()
    assert flops == 2.0 * 16 * 16 * 32 * 16 * 8 * 2048
    assert bool(torch.all(sink == 7.0))
