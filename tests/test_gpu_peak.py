"""The MFMA peak micro-benchmark (httm_peak_mfma) computes what its header
states: each lane's sum of its 8 chains, every chain accumulating, per group
of 8 iterations, A_j times B_((j + s) mod 8) for s = 0..7, with A and B the
pseudo-random bf16 operands the header defines, in the 16x16x32 MFMA lane
layout (A: row l%16, k = 8(l/16) + e; B: column l%16, same k; C: rows
4(l/16) + r, column l%16).  Compared with an fp64 product on the host; the
rate itself is a measurement, reported by bench.py."""
import numpy as np
import pytest

import token_merged_global_amd as H

pytestmark = pytest.mark.gpu


def _hash(x):
    x = x.astype(np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x7FEB352D) & 0xFFFFFFFF
    x ^= x >> 15
    x = (x * 0x846CA68B) & 0xFFFFFFFF
    x ^= x >> 16
    return x


def _bf16(x32):
    """Round fp32 values to bf16 (nearest, ties to even), returned as float64."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def _expected(grid, iters, a, b):
    n = grid * H.PEAK_THREADS
    g = np.arange(n, dtype=np.uint64)
    je = np.arange(64, dtype=np.uint64)
    h = _hash(g[:, None] * 64 + je[None, :])  # [lane][8 j + e]
    lo = ((h & 0xFFFF).astype(np.int64) - 32768).astype(np.float32) * np.float32(1.0 / 32768.0)
    hi = ((h >> 16).astype(np.int64) - 32768).astype(np.float32) * np.float32(1.0 / 32768.0)
    A = _bf16(np.float32(a) * lo).reshape(n // 64, 64, 8, 8)  # [wave][lane][j][e]
    B = _bf16(np.float32(b) * hi).reshape(n // 64, 64, 8, 8)
    out = np.empty((n // 64, 64))
    lanes = np.arange(64)
    for w in range(n // 64):
        # A_j[m][k] = A[w][m + 16 (k // 8)][j][k % 8]; B_p[k][n] = B[w][n + 16 (k // 8)][p][k % 8]
        Am = A[w].reshape(4, 16, 8, 8).transpose(2, 1, 0, 3).reshape(8, 16, 32)
        Bm = B[w].reshape(4, 16, 8, 8).transpose(2, 0, 3, 1).reshape(8, 32, 16)
        C = (iters // 8) * np.einsum("jmk,kn->jmn", Am, Bm.sum(axis=0))
        rows = 4 * (lanes // 16)[:, None] + np.arange(4)[None, :]
        out[w] = C[:, rows, (lanes % 16)[:, None]].sum(axis=(0, 2))
    return out.reshape(n), 32 * (iters // 8) * 8 * 8 * 4 * abs(a * b)


@pytest.mark.parametrize("iters,grid,a,b", [(8, 1, 1.0, 1.0), (64, 3, 0.5, 2.0), (800, 2, -1.0, 1.0)])
def test_peak_mfma_values(iters, grid, a, b):
    import torch
    n = grid * H.PEAK_THREADS
    out = torch.full((n + 512,), 7.0, dtype=torch.float32, device="cuda")
    flop = H.peak_mfma(iters, grid, out, a=a, b=b)
    torch.cuda.synchronize()
    assert flop == grid * iters * 4 * 8 * (2 * 16 * 16 * 32)
    want, bound = _expected(grid, iters, a, b)
    got = out.cpu().numpy().astype(np.float64)
    # fp32 accumulation of bf16 products: far below 1e-5 of the sum of |terms|
    assert np.abs(got[:n] - want).max() <= 1e-5 * bound, np.abs(got[:n] - want).max()
    assert (got[n:] == 7.0).all()


def test_peak_mfma_refuses_a_short_buffer():
    import torch
    out = torch.empty(255, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        H.peak_mfma(16, 1, out)
