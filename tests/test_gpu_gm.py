"""GPU parity of the head-shared global matching (partition = 2; the merging
the HTTM page contrasts itself with: one topology for every head from
global matching, research background and key designs 1-2) against the
oracle, staged: the head-mean metric bit for bit, matches and scores with
the near-tie rule, the top-r set and groups exactly, every head's query and
key groups the one shared partition, then deviations, outliers, the final
partition and outputs as for the other partitions."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from oracle import staged
import token_merged_global_amd as H
from gpu_util import BF16_REL, F32_ABS, bf16_to_f32, read_all, say, tile_rows, to_dev

pytestmark = pytest.mark.gpu


def _run(w, x, **kw):
    plan = H.Plan.from_workload(w, **kw)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    out = H.layer(plan, q, k, v, ws=ws)
    torch.cuda.synchronize()
    gpu = read_all(plan, ws, w.heads)
    if w.dtype == "bf16":
        gpu["gm_metric"] = bf16_to_f32(gpu["gm_metric"])
    return plan, ws, (q, k, v), out.float().cpu().numpy(), gpu


def _check(w, x, gpu, out, **kw):
    p = O.Params.from_workload(w)
    tol = dict(out_tol=F32_ABS) if w.dtype == "f32" else dict(rel_tol=BF16_REL)
    tol.update(kw)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, bf16=w.dtype == "bf16",
                             workers=gen.default_workers(), **tol)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
    return rep


def _small(**kw):
    return gen.WORKLOADS["vggt30"].with_(name="small", cfg_id=7, frames=6, heads=4, n_t=3, partition=2, **kw)


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1])
def test_gm_tiny_fp32(seed):
    w = gen.WORKLOADS["tiny"].with_(partition=2)
    say(f"[gm tiny fp32] seed={seed}")
    x = gen.layer_inputs(w, seed=seed)
    plan, ws, dev, out, gpu = _run(w, x)
    _check(w, x, gpu, out)


@pytest.mark.parametrize("kv", [0.0, 0.5, 0.75])
def test_gm_small_bf16_full_outputs(kv):
    """Merge ratios 0 (nothing merged), 0.5 and 0.75 (every source merges)."""
    w = _small(kv_ratio=kv)
    say(f"[gm small bf16] kv={kv} N={w.n_tokens}")
    x = gen.layer_inputs(w)
    plan, ws, dev, out, gpu = _run(w, x)
    P = w.frames * w.grid_h * w.grid_w
    r = min(P - (-(-P // 4)), int(np.floor(kv * P + 1e-9)))
    assert plan.info["kv_len"] == plan.info["q_groups"] == w.n_tokens - r
    _check(w, x, gpu, out)


def test_gm_vggt30():
    """30 frames x 1374 tokens, 16 heads: one shared partition from 30,810
    sources against 10,270 destinations; outputs of one token of every
    256-row query tile of two heads plus sampled tokens."""
    w = gen.WORKLOADS["vggt30"].with_(partition=2)
    x = gen.layer_inputs(w)
    plan, ws, dev, out, gpu = _run(w, x)
    oh = gen.oracle_heads(w)
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(w.n_tokens, 256, replace=False)] +
                                    [tile_rows(gpu["q_slot"][h], gpu["cu_q"], h) for h in oh]))
    say(f"[gm vggt30] rows {len(rows)}")
    _check(w, x, gpu, out, rows=rows, out_heads=oh)


@pytest.mark.parametrize("case", [dict(frames=1, grid_h=6, grid_w=7, n_special=1),
                                  dict(frames=9, grid_h=1, grid_w=1, n_special=3),
                                  dict(frames=5, grid_h=5, grid_w=7, n_special=2, heads=3)])
def test_gm_edge_geometry(case):
    """One frame, one patch per frame (a single destination per 4 frames), an
    odd grid: every index stage and every output row."""
    kw = dict(name="edge", cfg_id=22, dtype="bf16", heads=2, d_head=64, n_s=4, n_t=2, q_ratio=0.5,
              kv_ratio=0.5, outlier_pct=10.0, partition=2)
    kw.update(case)
    w = gen.Workload(**kw)
    say(f"[gm edge] {case}")
    x = gen.layer_inputs(w)
    plan, ws, dev, out, gpu = _run(w, x)
    _check(w, x, gpu, out, out_half_ulp=True)


def test_gm_repeat_cached_and_index_round_trip():
    """Repeat runs are bit-identical; cached layers on the shared indices
    match the oracle; an exported index drives identical cached layers."""
    w = _small()
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    o1, idx = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    o1 = o1.clone()
    o2 = H.layer(plan, q, k, v, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    gpu = read_all(plan, ws, w.heads, index=idx)
    qf = [staged.canonical(gpu["q_slot"][h]) for h in range(w.heads)]
    kr = [staged.canonical(gpu["kv_group"][h]) for h in range(w.heads)]
    assert all(np.array_equal(kr[0], kr[h]) for h in range(w.heads))
    x1 = gen.layer_inputs(w, layer=1)
    dev1 = [to_dev(x1[t], w.dtype) for t in "qkv"]
    c1 = H.layer_cached(plan, idx, *dev1, ws=ws).float().cpu().numpy()
    ref = O.layer_cached(x1["q"], x1["k"], x1["v"], O.Params.from_workload(w), qf, kr)
    err, rms = np.abs(c1 - ref).max(), np.sqrt((ref ** 2).mean())
    say(f"[gm cached] err {err:.3g} rms {rms:.3g}")
    assert err <= BF16_REL * rms
    host = H.index_export(plan, idx)
    c2 = H.layer_cached(plan, H.index_import(plan, host), *dev1, ws=ws)
    torch.cuda.synchronize()
    assert np.array_equal(c2.float().cpu().numpy(), c1)


@pytest.mark.timeout(600)
def test_gm_vggt100():
    """100 frames: the shared partition from 102,675 sources against 34,225
    destinations (every match staged on the CPU), deviations, outliers and
    the final partition of every head, sampled outputs of two heads."""
    w = gen.WORKLOADS["vggt100"].with_(partition=2)
    x = gen.layer_inputs(w)
    plan, ws, dev, out, gpu = _run(w, x)
    oh = gen.oracle_heads(w)
    rows = np.unique(np.r_[np.random.default_rng(6).choice(w.n_tokens, 256, replace=False), 0, w.n_tokens - 1])
    _check(w, x, gpu, out, rows=rows, out_heads=oh)
