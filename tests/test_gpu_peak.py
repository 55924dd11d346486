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


def _expected_fp8(grid, iters):
    """Lane sums of the FP8 micro-benchmark: e4m3 operands in the 32x32x64 MFMA
    lane layout (lane l, half h = l / 32: byte b < 16 is k = 16 h + b, byte
    b >= 16 is k = 32 + 16 h + b - 16; A row / B column l % 32; C rows
    8 (r / 4) + 4 h + r % 4 of column l % 32 in accumulator r)."""
    import torch
    n = grid * H.PEAK_THREADS
    g = np.arange(n, dtype=np.uint64)
    idx = g[:, None] * 128 + np.arange(64, dtype=np.uint64)[None, :]
    words = (_hash(idx) & 0xBFBFBFBF).astype(np.uint32)  # [lane][16 j + w]: A_j words 0-7, B_j words 8-15
    byts = words.view(np.uint8).reshape(n, 4, 2, 32)  # [lane][j][A or B][byte]
    vals = torch.from_numpy(np.ascontiguousarray(byts)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    b = np.arange(32)
    out = np.empty((n // 64, 64))
    lanes = np.arange(64)
    h = lanes // 32
    kmap = np.where(b[None, :] < 16, 16 * h[:, None] + b[None, :], 32 + 16 * h[:, None] + b[None, :] - 16)  # [lane][byte]
    for w in range(n // 64):
        A = np.zeros((4, 32, 64))
        Bm = np.zeros((4, 64, 32))
        for l in range(64):
            A[:, l % 32, kmap[l]] = vals[64 * w + l, :, 0, :]
            Bm[:, kmap[l], l % 32] = vals[64 * w + l, :, 1, :]
        C = (iters // 4) * np.einsum("jmk,kn->jmn", A, Bm.sum(axis=0))
        r = np.arange(16)
        rows = 8 * (r // 4)[None, :] + 4 * h[:, None] + (r % 4)[None, :]  # [lane][r]
        out[w] = C[:, rows, (lanes % 32)[:, None]].sum(axis=(0, 2))
    return out.reshape(n), (iters // 4) * 4 * 4 * 16 * 64 * 1.875 ** 2


@pytest.mark.parametrize("iters,grid", [(4, 1), (64, 2)])
def test_peak_mfma_fp8_values(iters, grid):
    import torch
    n = grid * H.PEAK_THREADS
    out = torch.full((n + 512,), 7.0, dtype=torch.float32, device="cuda")
    flop = H.peak_mfma_fp8(iters, grid, out)
    torch.cuda.synchronize()
    assert flop == grid * iters * 4 * 4 * (2 * 32 * 32 * 64)
    want, bound = _expected_fp8(grid, iters)
    got = out.cpu().numpy().astype(np.float64)
    assert np.abs(got[:n] - want).max() <= 1e-5 * bound, np.abs(got[:n] - want).max()
    assert (got[n:] == 7.0).all()
