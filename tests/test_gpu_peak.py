"""The MFMA peak micro-benchmark (httm_peak_mfma) computes what it states:
every lane ends with 1024 * a * b * iters, exactly, and nothing past the
grid's lanes is written.  Its rate is a measurement, checked by bench.py,
not here."""
import pytest

import token_merged_global_amd as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("iters,grid,a,b", [(1, 1, 1.0, 1.0), (1000, 8, 0.5, 3.0), (4000, 300, -0.25, 2.0)])
def test_peak_mfma_values(iters, grid, a, b):
    import torch
    n = grid * H.PEAK_THREADS
    out = torch.full((n + 512,), 7.0, dtype=torch.float32, device="cuda")
    flop = H.peak_mfma(iters, grid, out, a=a, b=b)
    torch.cuda.synchronize()
    assert flop == grid * iters * 4 * 8 * (2 * 16 * 16 * 32)
    want = 1024.0 * a * b * iters
    assert abs(want) < 2 ** 24
    got = out.cpu()
    assert bool((got[:n] == want).all()), (got[:n].min().item(), got[:n].max().item(), want)
    assert bool((got[n:] == 7.0).all())


def test_peak_mfma_refuses_a_short_buffer():
    import torch
    out = torch.empty(255, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        H.peak_mfma(10, 1, out)
