"""GPU parity at the full VGGT-shaped sizes: 100 frames, the 200-frame sweep,
and the 500-frame six-layer stack with cached merge indices.

Index stages (matches, top-r groups, deviations, the global outlier choice,
the final query partition) are checked on every head against the oracle;
outputs on sampled rows of the seeded oracle heads (the oracle computes one
output row from that row's query slot and all merged keys), within 2e-2 x RMS.
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from oracle import staged
import token_merged_global_amd as H
from gpu_util import BF16_REL, read_all, run_layer, sample_rows, say, tile_rows, to_dev

pytestmark = pytest.mark.gpu
WORKERS = gen.default_workers()


def _rows(w, gpu, rows_seed):
    """256 sampled tokens plus one token of every 256-row query tile of the
    oracle heads (every attention work unit of those heads is checked)."""
    oh = gen.oracle_heads(w)
    tiles = [tile_rows(gpu["q_slot"][h], gpu["cu_q"], h) for h in oh]
    return np.unique(np.concatenate([sample_rows(w.n_tokens, 256, rows_seed)] + tiles))


def _check(w, x, gpu, out, p=None, rows_seed=0):
    p = p or O.Params.from_workload(w)
    oh = gen.oracle_heads(w)
    rows = _rows(w, gpu, rows_seed)
    say(f"   output rows checked per oracle head: {len(rows)}")
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, out_heads=oh, rows=rows,
                             rel_tol=BF16_REL, workers=WORKERS)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
    return rep


@pytest.mark.timeout(600)
def test_vggt100_layer():
    w = gen.WORKLOADS["vggt100"]
    say(f"[vggt100] N={w.n_tokens}")
    x = gen.layer_inputs(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    _check(w, x, gpu, out)
    cu = gpu["cu_q"]
    assert cu[-1] <= plan.info["q_capacity"]


@pytest.mark.timeout(900)
def test_vggt200_sweep_and_ratio_zero():
    """K/V merge {0.5, 0.75} x outlier {5, 10, 20} %, every point staged against
    the oracle, plus merge ratio 0."""
    w = gen.WORKLOADS["vggt200"]
    say(f"[vggt200] N={w.n_tokens}")
    x = gen.layer_inputs(w)
    masks = {}
    for kv in (0.5, 0.75):
        for pct in (5.0, 10.0, 20.0):
            wk = w.with_(kv_ratio=kv, outlier_pct=pct)
            plan, ws, dev, out, gpu, _ = run_layer(wk, x)
            say(f"  kv={kv} p={pct}: q_len/head={np.diff(gpu['cu_q']).mean():.0f} kv_len={plan.info['kv_len']}")
            assert int(gpu["outlier"].sum()) == plan.info["n_outliers"]
            masks[(kv, pct)] = gpu["outlier"].astype(bool)
            _check(wk, x, gpu, out, rows_seed=int(pct))
            del ws, dev
            torch.cuda.empty_cache()
    # nesting: a larger budget keeps every earlier outlier (same query groups)
    for kv in (0.5, 0.75):
        assert not (masks[(kv, 5.0)] & ~masks[(kv, 10.0)]).any()
        assert not (masks[(kv, 10.0)] & ~masks[(kv, 20.0)]).any()
        # queries do not depend on the key merge
    assert np.array_equal(masks[(0.5, 10.0)], masks[(0.75, 10.0)])
    # merge ratio 0: exact attention on sampled rows of two heads
    w0 = w.with_(q_ratio=0.0, kv_ratio=0.0)
    plan, ws, dev, out, gpu, _ = run_layer(w0, x)
    assert (np.diff(gpu["cu_q"]) == w.n_tokens).all()
    rows = sample_rows(w.n_tokens, 128, 7)
    for h in gen.oracle_heads(w):
        ref = O.attention(x["q"][h][rows], x["k"][h], x["v"][h], 0.125)
        err = np.abs(out[h][rows] - ref).max()
        say(f"  ratio 0 head {h}: err {err:.3g} rms {np.sqrt((ref ** 2).mean()):.3g}")
        assert err <= BF16_REL * np.sqrt((ref ** 2).mean())


@pytest.mark.timeout(900)
def test_vggt500_cached_stack():
    """Layer 0 computes the merge indices; layers 1-5 reuse them.

    Cached layers are independent across heads (no cross-head step), so the
    two oracle heads get their exact layer-l inputs and the other heads keep
    their layer-0 values; only the oracle heads' outputs are compared.
    """
    w = gen.WORKLOADS["vggt500"]
    oh = gen.oracle_heads(w)
    say(f"[vggt500] N={w.n_tokens} oracle heads {oh}")
    x0 = gen.layer_inputs(w)
    plan, ws, dev, out0, gpu, idx = run_layer(w, x0, keep_index=True)
    _check(w, x0, gpu, out0)
    qf = {h: staged.canonical(gpu["q_slot"][h]) for h in oh}
    kr = {h: staged.canonical(gpu["kv_group"][h]) for h in oh}
    stack_rows = _rows(w, gpu, 11)
    q, k, v = dev
    del out0, gpu
    p = O.Params.from_workload(w)
    rows = stack_rows
    say(f"   cached layers: output rows checked per oracle head: {len(rows)}")
    for l, xl in gen.layer_stack(w, heads=oh):
        if l == 0:
            continue
        for t, d in zip("qkv", (q, k, v)):
            for i, h in enumerate(oh):
                d[h].copy_(to_dev(xl[t][i], w.dtype))
        out = H.layer_cached(plan, idx, q, k, v, ws=ws).float().cpu().numpy()
        for i, h in enumerate(oh):
            ref = O.layer_cached(xl["q"][i:i + 1], xl["k"][i:i + 1], xl["v"][i:i + 1], p, [qf[h]], [kr[h]],
                                 rows=rows)[0]
            err = np.abs(out[h][rows] - ref).max()
            rms = np.sqrt((ref ** 2).mean())
            say(f"  layer {l} head {h}: err {err:.3g} rms {rms:.3g}")
            assert err <= BF16_REL * rms


@pytest.mark.timeout(600)
def test_vggt100_geometry_aware_layer():
    """The geometry-aware partition at 100 frames (137,400 tokens): variance
    map, classes and groups of every head and stream; the global match (about
    86,500 sources against 36,700 destinations per head and stream) against
    the oracle on two heads; deviations, the outlier choice and the final
    partition on every head; outputs on sampled rows of the oracle heads."""
    w = gen.WORKLOADS["vggt100"].with_(partition=1, protect_pct=10.0)
    say(f"[vggt100 geometry-aware] N={w.n_tokens}")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    oh = gen.oracle_heads(w)
    rows = sample_rows(w.n_tokens, 256, 1)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, out_heads=oh, rows=rows, rel_tol=BF16_REL,
                             match_heads=[0, w.heads - 1], workers=WORKERS)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
    kl = gpu["kv_len"]
    assert (kl <= plan.info["kv_len"]).all()


@pytest.mark.timeout(900)
def test_largest_head_at_the_offset_limit():
    """One head of 4,095 frames x 64x64 patches (N = 16,773,120, just under the
    2^24 limit) with no key merge: the head's K~ and V~^T span just under 2^31
    bytes, the end of the attention kernels' 32-bit buffer offsets.  Index
    stages on the whole head against the oracle, outputs on sampled rows."""
    w = gen.WORKLOADS["vggt30"].with_(name="maxhead", cfg_id=12, heads=1, frames=4095, grid_h=64, grid_w=64,
                                      n_special=0, n_s=128, n_t=30, kv_ratio=0.0)
    assert w.n_tokens == 16773120
    say(f"[maxhead] N={w.n_tokens}")
    x = gen.layer_inputs(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    assert plan.info["kv_len"] == w.n_tokens
    del ws, dev
    torch.cuda.empty_cache()
    rows = np.unique(np.r_[sample_rows(w.n_tokens, 48, 5), np.arange(w.n_tokens - 64, w.n_tokens, 16)])
    rep = staged.check_layer(x["q"], x["k"], x["v"], O.Params.from_workload(w), gpu, out, rows=rows,
                             rel_tol=BF16_REL, workers=WORKERS)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
