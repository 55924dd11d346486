"""Helpers shared by the GPU parity tests (marshalling only)."""
import sys

import numpy as np
import torch

import token_merged_global_amd as H

BF16_REL = 2e-2  # outputs: max-abs error <= 2e-2 * RMS(oracle output) for bf16
F32_ABS = 1e-4   # outputs: max-abs error <= 1e-4 for fp32
PER_HEAD = ["q_match", "q_score", "kv_match", "kv_score", "q_group", "kv_group", "delta", "outlier", "q_slot"]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def read_all(plan, ws, heads, index=None):
    gpu = {it: H.debug_read(plan, ws, it, index=index) for it in H.debug_items(plan)}
    for it in PER_HEAD:
        if it in gpu:
            gpu[it] = gpu[it].reshape(heads, -1)
    return gpu


def run_layer(w, inputs, keep_index=False, **plan_kw):
    plan = H.Plan.from_workload(w, **plan_kw)
    q, k, v = (to_dev(inputs[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    res = H.layer(plan, q, k, v, ws=ws, keep_index=keep_index)
    out, idx = (res if keep_index else (res, None))
    torch.cuda.synchronize()
    gpu = read_all(plan, ws, w.heads, index=idx)
    o = out.float().cpu().numpy()
    del out
    return plan, ws, (q, k, v), o, gpu, idx


def sample_rows(n, count, seed):
    rows = np.random.default_rng(seed).choice(n, count, replace=False)
    return np.unique(np.r_[rows, [0, 1, n - 1]])


def tile_rows(q_slot_h: np.ndarray, cu_q: np.ndarray, h: int, tile: int = 256) -> np.ndarray:
    """One token per `tile`-row query tile of head h: the token whose packed
    row is the first one at or after the tile's start (every packed row has
    at least one token)."""
    order = np.argsort(q_slot_h, kind="stable")
    srt = q_slot_h[order]
    starts = np.arange(cu_q[h], cu_q[h + 1], tile)
    pos = np.searchsorted(srt, starts)
    assert (pos < len(srt)).all() and (srt[pos] < cu_q[h + 1]).all()
    return np.unique(order[pos])


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def segment_means(x: np.ndarray, label: np.ndarray, n_seg: int) -> np.ndarray:
    """fp64 mean of the rows of x sharing each label in [0, n_seg) (label -1: skipped)."""
    keep = label >= 0
    s = np.zeros((n_seg, x.shape[1]), np.float64)
    np.add.at(s, label[keep], x[keep].astype(np.float64))
    c = np.bincount(label[keep], minlength=n_seg).astype(np.float64)
    assert (c > 0).all()
    return s / c[:, None]
