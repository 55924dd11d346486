"""GPU parity of the HIP layer against the CPU oracle (staged; see oracle/staged.py).

Tolerances (stated by the benchmark spec): index sets bit-exact apart from
counted near-ties (|dsim| < 1e-5); outputs within 1e-4 max-abs for fp32 and
within 2e-2 * RMS(oracle output) max-abs for bf16.  Deviations and outlier
masks are checked bit-exactly on the GPU's own groups.
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from oracle import staged
import token_merged_global_amd as H

pytestmark = pytest.mark.gpu

from gpu_util import BF16_REL, F32_ABS, bf16_to_f32, read_all, say as _say, segment_means, to_dev


def run_layer(w, inputs, **plan_kw):
    plan = H.Plan.from_workload(w, **plan_kw)
    q, k, v = (to_dev(inputs[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    out = H.layer(plan, q, k, v, ws=ws)
    torch.cuda.synchronize()
    return plan, ws, (q, k, v), out.float().cpu().numpy(), read_all(plan, ws, w.heads)


def small_bf16(frames=6, heads=4, n_t=3, **kw):
    return gen.WORKLOADS["vggt30"].with_(name="small", cfg_id=7, frames=frames, heads=heads, n_t=n_t, **kw)


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1, gen.DEFAULT_SEED + 2])
def test_tiny_fp32_layer(seed):
    w = gen.WORKLOADS["tiny"]
    _say(f"[tiny fp32] seed={seed}")
    x = gen.layer_inputs(w, seed=seed)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, out_tol=F32_ABS)
    _say("  ", rep.as_dict())
    # unstaged: the oracle's own indices, when no near-tie occurred
    if rep.match_near_ties == 0 and rep.select_near_ties == 0:
        tr = O.layer(x["q"], x["k"], x["v"], p)
        assert np.abs(out - tr.out).max() <= F32_ABS
    assert rep.delta_nonexact == 0


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1])
def test_small_bf16_layer_full_outputs(seed):
    w = small_bf16()
    _say(f"[small bf16] seed={seed} N={w.n_tokens}")
    x = gen.layer_inputs(w, seed=seed)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1, gen.DEFAULT_SEED + 2])
def test_vggt30_layer(seed):
    """30 frames x 1374 tokens, 16 heads: every index stage on all heads, sampled outputs."""
    w = gen.WORKLOADS["vggt30"]
    _say(f"[vggt30] seed={seed}")
    x = gen.layer_inputs(w, seed=seed)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    rows = np.sort(np.random.default_rng(seed).choice(w.n_tokens, 384, replace=False))
    rows = np.unique(np.r_[rows, [0, 1, 4, w.n_tokens - 1]])
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rows=rows, rel_tol=BF16_REL)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
    cu = gpu["cu_q"]
    assert cu[0] == 0 and cu[-1] <= plan.info["q_capacity"]
    assert (np.diff(cu) <= plan.info["q_groups"] + plan.info["n_outliers"]).all()


def test_xcd_tail_tiles_full_outputs():
    """A layer whose 256-row query tiles leave partly filled last rounds on the
    XCDs: tail tiles run with twice the key splits and a separate partial-row
    region; every output row is checked against the oracle."""
    w = small_bf16(frames=8, heads=16)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    tiles = int(sum(-(-int(n) // 256) for n in np.diff(gpu["cu_q"])))
    shares = [(i + 1) * tiles // 8 - i * tiles // 8 for i in range(8)]
    _say(f"[xcd tail] tiles={tiles} per-XCD={shares}")
    # 16 tiles per full round of an XCD on gfx950 (2 workgroups x 32 CUs, 4 splits)
    assert any(n > 16 and n % 16 for n in shares)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


@pytest.mark.parametrize("name", ["tiny", "small", "vggt30"])
def test_frame_minor_blocks(name):
    """block_order = 1: frames vary fastest inside a block (the alternative
    stacking of the HTTM page's temporal reordering); staged parity as for
    frame-major blocks."""
    w = {"tiny": gen.WORKLOADS["tiny"], "small": small_bf16(), "vggt30": gen.WORKLOADS["vggt30"]}[name]
    w = w.with_(block_order=1)
    _say(f"[frame-minor] {name}")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    assert p.block_order == 1
    plan, ws, dev, out, gpu = run_layer(w, x)
    kw = {"out_tol": F32_ABS} if w.dtype == "f32" else {"rel_tol": BF16_REL}
    if name == "vggt30":
        rows = np.unique(np.r_[np.random.default_rng(5).choice(w.n_tokens, 256, replace=False), 0, w.n_tokens - 1])
        kw["rows"] = rows
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, **kw)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


def test_ratio_zero_is_exact_attention():
    w = small_bf16(frames=4, heads=2, q_ratio=0.0, kv_ratio=0.0)
    x = gen.layer_inputs(w)
    plan, ws, (q, k, v), out, gpu = run_layer(w, x)
    assert (np.diff(gpu["cu_q"]) == w.n_tokens).all()
    for h in range(w.heads):
        ref = O.attention(x["q"][h], x["k"][h], x["v"][h], 0.125)
        rms = np.sqrt((ref ** 2).mean())
        assert np.abs(out[h] - ref).max() <= BF16_REL * rms
    dense = H.attention_dense(plan, q, k, v).float().cpu().numpy()
    for h in range(w.heads):
        ref = O.attention(x["q"][h], x["k"][h], x["v"][h], 0.125)
        assert np.abs(dense[h] - ref).max() <= BF16_REL * np.sqrt((ref ** 2).mean())


def test_outlier_100_keeps_every_query():
    w = small_bf16(frames=4, heads=2, outlier_pct=100.0)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    assert gpu["outlier"].all()
    assert (np.diff(gpu["cu_q"]) == w.n_tokens).all()
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    _say("  ", rep.as_dict())


def test_dense_attention_fp32_and_bf16():
    for dtype in ["f32", "bf16"]:
        w = small_bf16(frames=2, heads=2).with_(dtype=dtype)
        x = gen.layer_inputs(w)
        plan = H.Plan.from_workload(w)
        q, k, v = (to_dev(x[t], dtype) for t in "qkv")
        out = H.attention_dense(plan, q, k, v).float().cpu().numpy()
        for h in range(w.heads):
            ref = O.attention(x["q"][h], x["k"][h], x["v"][h], 0.125)
            err = np.abs(out[h] - ref).max()
            tol = F32_ABS if dtype == "f32" else BF16_REL * np.sqrt((ref ** 2).mean())
            _say(f"[dense {dtype}] head {h} err {err:.3g} tol {tol:.3g}")
            assert err <= tol


def test_repeat_runs_are_bit_identical():
    w = small_bf16(frames=4, heads=3)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    o1 = H.layer(plan, q, k, v, ws=ws).clone()
    d1 = {it: H.debug_read(plan, ws, it) for it in H.debug_items(plan)}
    o2 = H.layer(plan, q, k, v, ws=ws)
    d2 = {it: H.debug_read(plan, ws, it) for it in H.debug_items(plan)}
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for it in d1:
        assert np.array_equal(d1[it], d2[it]), it


def test_cached_layer_matches_oracle_with_same_indices():
    w = small_bf16(frames=6, heads=2)
    x0 = gen.layer_inputs(w)
    x1 = {t: gen.round_bf16(x0[t] + np.random.default_rng(5).normal(0, 0.02, x0[t].shape).astype(np.float32))
          for t in "qkv"}
    p = O.Params.from_workload(w)
    plan = H.Plan.from_workload(w)
    dev0 = [to_dev(x0[t], w.dtype) for t in "qkv"]
    dev1 = [to_dev(x1[t], w.dtype) for t in "qkv"]
    ws = H.workspace(plan)
    out0, idx = H.layer(plan, *dev0, ws=ws, keep_index=True)
    torch.cuda.synchronize()
    q_slot = H.debug_read(plan, ws, "q_slot", index=idx).reshape(w.heads, -1)
    kv_group = H.debug_read(plan, ws, "kv_group").reshape(w.heads, -1)
    out1 = H.layer_cached(plan, idx, *dev1, ws=ws).float().cpu().numpy()
    qf = [staged.canonical(q_slot[h]) for h in range(w.heads)]
    kr = [staged.canonical(kv_group[h]) for h in range(w.heads)]
    ref = O.layer_cached(x1["q"], x1["k"], x1["v"], p, qf, kr)
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(out1 - ref).max()
    _say(f"[cached] err {err:.3g} rms {rms:.3g}")
    assert err <= BF16_REL * rms
    # an index from another plan is refused
    other = H.Plan.from_workload(w)
    with pytest.raises(H.HttmError):
        H.layer_cached(other, idx, *dev1)


def _orthogonal_offset(x, big=600.0):
    """Keys confined to channels 0-31; queries get a large constant in channels
    32-63, orthogonal to every key.  Scores (and the softmax) are unchanged in
    size, but the norm bound |q| max|k| exceeds every score by far more than
    60 (log2 units), so every attention unit takes the exact path."""
    q = x["q"].copy()
    k = x["k"].copy()
    k[..., 32:] = 0.0
    q[..., 32:] = big
    return {"q": gen.round_bf16(q), "k": gen.round_bf16(k), "v": x["v"]}


def test_attention_fallback_exact_path():
    w = small_bf16(frames=4, heads=2)
    xs = _orthogonal_offset(gen.layer_inputs(w))
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, xs)
    fb = int(gpu["attn_fallback"][0])
    _say(f"[fallback] units recomputed exactly: {fb}")
    assert fb > 0
    rep = staged.check_layer(xs["q"], xs["k"], xs["v"], p, gpu, out, rel_tol=BF16_REL)
    _say("  ", rep.as_dict())
    # the unmerged path takes the same fallback
    q, k, v = dev
    dense = H.attention_dense(plan, q, k, v).float().cpu().numpy()
    for h in range(w.heads):
        ref = O.attention(xs["q"][h], xs["k"][h], xs["v"][h], 0.125)
        assert np.abs(dense[h] - ref).max() <= BF16_REL * np.sqrt((ref ** 2).mean())


@pytest.mark.parametrize("split", [1, 2, 4, 8])
def test_attention_key_splits_against_oracle(split):
    """Attention with its keys split in 1, 2, 4 or 8 ranges (partials combined
    in a fixed order) against the oracle on every output row of a layer with
    several query tiles per head and partly filled last rounds on the XCDs."""
    w = small_bf16(frames=8, heads=16)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x, attn_split=split)
    _say(f"[split {split}] q rows per head {np.diff(gpu['cu_q']).tolist()[:4]}...")
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    _say("  ", rep.as_dict())


def _merged_rows_check(plan, ws, w, x, gpu, what):
    """Every merged key, value and query row against the fp64 mean of its
    members (the group the implementation formed), within one rounding of
    the stored type (bf16: 2^-8 relative, fp32: 1e-6 relative)."""
    h, N = w.heads, w.n_tokens
    lkp = -(-plan.info["kv_len"] // 64) * 64
    lk = plan.info["kv_len"]
    conv = bf16_to_f32 if w.dtype == "bf16" else (lambda a: a)
    kt = conv(H.debug_read(plan, ws, "kt")).reshape(h, lkp, 64)
    vt = conv(H.debug_read(plan, ws, "vt")).reshape(h, 64, lkp)
    qt = conv(H.debug_read(plan, ws, "qt")).reshape(-1, 64)
    rel = 2.0 ** -8 if w.dtype == "bf16" else 1e-6
    kscale = plan.info["softmax_scale"] * 1.4426950408889634
    cu = gpu["cu_q"]
    worst = 0.0
    for i in range(h):
        km = segment_means(x["k"][i], gpu["kv_group"][i], lk) * kscale
        vm = segment_means(x["v"][i], gpu["kv_group"][i], lk)
        qm = segment_means(x["q"][i], gpu["q_slot"][i] - cu[i], cu[i + 1] - cu[i])
        for got, ref in ((kt[i, :lk], km), (vt[i, :, :lk].T, vm), (qt[cu[i]:cu[i + 1]], qm)):
            err = np.abs(got - ref) - rel * np.abs(ref) - 2e-6  # + fp32 summation error of the mean
            worst = max(worst, float((np.abs(got - ref) / (np.abs(ref) + 1e-3)).max()))
            assert (err <= 0).all(), f"{what} head {i}: merged row off by {np.abs(got - ref).max():.3g}"
        assert (kt[i, lk:] == 0).all() and (vt[i, :, lk:] == 0).all()
    _say(f"[merged rows {what}] worst relative error {worst:.3g}")


@pytest.mark.parametrize("name", ["tiny", "small", "vggt30"])
def test_merged_rows_are_group_means(name):
    """K~ (times scale * log2 e), V~ (transposed) and the packed Q~ rows read
    back and compared with the fp64 means of their groups (HTTM page, key
    design 1: a merged token is the mean of its members, V follows K's
    groups; key design 3: outliers leave their group and become rows of
    their own); then again after a cached layer on new inputs (LiteVGGT
    page, key design 3: reused indices, recomputed means)."""
    w = {"tiny": gen.WORKLOADS["tiny"], "small": small_bf16(), "vggt30": gen.WORKLOADS["vggt30"]}[name]
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    _, idx = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    torch.cuda.synchronize()
    gpu = read_all(plan, ws, w.heads, index=idx)
    _merged_rows_check(plan, ws, w, x, gpu, f"{name} layer")
    x1 = gen.layer_inputs(w, layer=1)
    for t, d in zip("qkv", (q, k, v)):
        d.copy_(to_dev(x1[t], w.dtype))
    H.layer_cached(plan, idx, q, k, v, ws=ws)
    torch.cuda.synchronize()
    _merged_rows_check(plan, ws, w, x1, gpu, f"{name} cached layer")


def test_vggt30_every_query_slot():
    """30 frames, 16 heads: after the staged index checks, the output of one
    token of every merged query row of every head (about 8,400 per head)
    against the oracle's attention on the implementation's partitions."""
    w = gen.WORKLOADS["vggt30"]
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    rows = np.unique(np.r_[np.random.default_rng(3).choice(w.n_tokens, 64, replace=False), 0, w.n_tokens - 1])
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rows=rows, rel_tol=BF16_REL,
                             workers=gen.default_workers())
    _say("  ", rep.as_dict())
    worst = 0.0
    for h in range(w.heads):
        qf = staged.canonical(gpu["q_slot"][h])
        kr = staged.canonical(gpu["kv_group"][h])
        reps = np.unique(qf)  # one token per final query slot
        ref = O.head_output(x["q"][h], x["k"][h], x["v"][h], qf, kr, p.scale, rows=reps)
        rms = float(np.sqrt((ref ** 2).mean()))
        err = float(np.abs(out[h][reps] - ref).max())
        worst = max(worst, err / rms)
        assert err <= BF16_REL * rms, f"head {h}: {err:.3g} > {BF16_REL} x {rms:.3g}"
        assert len(reps) == gpu["cu_q"][h + 1] - gpu["cu_q"][h]
    _say(f"[vggt30 every slot] worst error / RMS {worst:.4f}")


def test_call_on_another_stream_without_workspace():
    """A layer enqueued on a stream that is not the current one, with no
    workspace passed: the temporary workspace and the output come from that
    stream's allocations, so tensors allocated right afterwards on the
    current stream cannot take them over while the layer runs."""
    w = small_bf16(frames=6, heads=4)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ref = H.layer(plan, q, k, v, ws=H.workspace(plan))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        o = H.layer(plan, q, k, v, stream=s)
        junk = torch.full((plan.workspace_bytes // 4 + 1024,), 7.0, device="cuda")  # current stream
        outs.append(o)
        del junk
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))


def test_index_export_import_round_trip():
    """Cached indices through host memory (LiteVGGT page, key design 3): an
    exported index, imported into a fresh buffer or by another plan with the
    same parameters, drives bit-identical cached layers; bytes from other
    parameters or with out-of-range contents are refused."""
    w = small_bf16(frames=4, heads=3)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    _, idx = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    host = H.index_export(plan, idx)
    assert host.nbytes == plan.index_bytes
    o1 = H.layer_cached(plan, idx, q, k, v, ws=ws).clone()
    o2 = H.layer_cached(plan, H.index_import(plan, host), q, k, v, ws=ws).clone()
    plan_b = H.Plan.from_workload(w)
    o3 = H.layer_cached(plan_b, H.index_import(plan_b, host), q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    # other parameters (same index size): header mismatch
    plan_c = H.Plan.from_workload(w.with_(outlier_pct=5.0))
    if plan_c.index_bytes == plan.index_bytes:
        with pytest.raises(H.HttmError) as e:
            H.index_import(plan_c, host)
        assert e.value.status == 4
    # a token id out of range after a valid header (the first member list
    # starts at the first 256-byte boundary after the 64-byte header)
    bad = host.copy()
    bad.view(np.int32)[256 // 4] = w.n_tokens
    with pytest.raises(H.HttmError) as e:
        H.index_import(plan, bad)
    assert e.value.status == 4


@pytest.mark.parametrize("dtype,order,qs,ks", [("bf16", 0, 0, 0), ("f32", 0, 0, 0), ("bf16", 1, 5, 3),
                                               ("f32", 1, 0, 6)])
def test_odd_geometry_layer(dtype, order, qs, ks):
    """A grid whose runs and temporal groups do not divide evenly (5 x 9
    patches, runs of 10, groups of 3 over 7 frames, 2 specials), explicit
    destination strides and both stacking orders: every index stage and
    every output row against the oracle."""
    w = gen.Workload(name="odd", cfg_id=9, dtype=dtype, heads=3, d_head=64, frames=7, grid_h=5, grid_w=9,
                     n_special=2, n_s=10, n_t=3, q_ratio=0.6, kv_ratio=0.3, outlier_pct=7.5, block_order=order,
                     q_dst_stride=qs, kv_dst_stride=ks)
    _say(f"[odd geometry] {dtype} order {order} strides {qs}/{ks}")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    kw = dict(rel_tol=BF16_REL) if dtype == "bf16" else dict(out_tol=F32_ABS)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, **kw)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


EDGE_CASES = {
    # one frame: a single temporal group shorter than n_t
    "one_frame": dict(frames=1, grid_h=6, grid_w=6, n_special=1, n_s=12, n_t=4),
    # runs longer than a frame (one spatial run per frame)
    "run_covers_frame": dict(frames=5, grid_h=3, grid_w=4, n_special=2, n_s=64, n_t=2),
    # one patch per frame
    "one_patch": dict(frames=9, grid_h=1, grid_w=1, n_special=3, n_s=1, n_t=4),
    # no outliers, keys unmerged, queries merged
    "no_outliers_kv0": dict(frames=4, grid_h=5, grid_w=5, n_special=0, n_s=10, n_t=2, outlier_pct=0.0,
                            kv_ratio=0.0),
    # queries unmerged, keys merged hard
    "q0_kv90": dict(frames=4, grid_h=5, grid_w=5, n_special=1, n_s=25, n_t=4, q_ratio=0.0, kv_ratio=0.9),
    # many heads of a small layer
    "heads64": dict(heads=64, frames=2, grid_h=3, grid_w=3, n_special=1, n_s=9, n_t=2),
    # the largest block with explicit stride 2 for keys (2048 destinations: more than the block-resident
    # similarity holds in LDS, so that stream takes the per-chunk kernel) and the derived stride 4 for
    # queries (1024 destinations: the most the block-resident kernel holds)
    "block4096_strides_4_2": dict(heads=1, frames=2, grid_h=64, grid_w=64, n_special=1, n_s=4096, n_t=1,
                                  q_ratio=0.5, kv_ratio=0.5, kv_dst_stride=2),
    # the largest block (4096 tokens: one 64 x 64 frame) and the largest stride (merge 95 %)
    "max_block": dict(heads=1, frames=2, grid_h=64, grid_w=64, n_special=1, n_s=4096, n_t=1, q_ratio=0.95,
                      kv_ratio=0.75),
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", sorted(EDGE_CASES))
def test_edge_geometry_layers(case, dtype):
    """Degenerate shapes of the method: every index stage and every output
    row against the oracle."""
    kw = dict(name="edge", cfg_id=21, dtype=dtype, heads=2, d_head=64, q_ratio=0.5, kv_ratio=0.5,
              outlier_pct=10.0)
    kw.update(EDGE_CASES[case])
    w = gen.Workload(**kw)
    _say(f"[edge] {case} {dtype} N={w.n_tokens}")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu = run_layer(w, x)
    # these tiny layers have outputs up to 7 x their RMS, where rounding the
    # output to bf16 alone can exceed 2e-2 x RMS: half an ulp of the largest
    # output is allowed on top (bf16 only)
    tol = dict(rel_tol=BF16_REL, out_half_ulp=True) if dtype == "bf16" else dict(out_tol=F32_ABS)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, **tol)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


@pytest.mark.parametrize("variant", ["f32", "bf16", "fp8"])
def test_degenerate_values(variant):
    """Zero and extreme-magnitude tokens.  Head 0: every query and key is zero
    (every cosine is 0, so ties alone decide matches and selection; every
    deviation is 0; attention is uniform over the merged keys).  Head 1: keys
    scaled by 2^-40 and queries by 2^40 (norms far from 1; with FP8 scores,
    scale exponents far from 0).  Index stages and every output row against
    the oracle."""
    dtype = "f32" if variant == "f32" else "bf16"
    w = gen.WORKLOADS["vggt30"].with_(name="degenerate", cfg_id=22, frames=4, heads=3, n_t=2, dtype=dtype,
                                      attn_fp8=(variant == "fp8"))
    x = gen.layer_inputs(w)
    x["q"][0] = 0.0
    x["k"][0] = 0.0
    x["q"][1] *= np.float32(2.0 ** 40)
    x["k"][1] *= np.float32(2.0 ** -40)
    p = O.Params.from_workload(w)
    _say(f"[degenerate] {variant} N={w.n_tokens}")
    plan, ws, dev, out, gpu = run_layer(w, x)
    assert np.isfinite(out).all()
    tol = dict(rel_tol=BF16_REL) if dtype == "bf16" else dict(out_tol=F32_ABS)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, **tol)
    _say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


def test_serial_timing_mode_is_bit_identical():
    """With the serialized timing mode every launch of a layer (and a cached
    layer) goes to the caller's stream: the same kernels on the same data, so
    the same bits as the forked schedule."""
    w = small_bf16(frames=6, heads=4)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    o1, idx = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    c1 = H.layer_cached(plan, idx, q, k, v, ws=ws)
    o1, c1 = o1.clone(), c1.clone()
    H.set_timing(None, serial=True)
    try:
        o2 = H.layer(plan, q, k, v, ws=ws, index=idx)
        c2 = H.layer_cached(plan, idx, q, k, v, ws=ws)
        torch.cuda.synchronize()
        stages, calls = H.get_timing()
    finally:
        H.set_timing([])
    assert calls == 2 and stages["sim_k"] > 0 and stages["merge_kv"] > 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_forced_launch_failure_then_normal_calls():
    """The error path part way through a layer (test hook): the n-th launch
    reports HTTM_ERR_DEVICE, the call returns that status, and the following
    calls on the same buffers run normally, bit-identical to before."""
    w = small_bf16(frames=4, heads=2)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    ref = H.layer(plan, q, k, v, ws=ws).clone()
    try:
        for n in (1, 3, 7):
            H.debug_fail_launch(n)
            with pytest.raises(H.HttmError) as e:
                H.layer(plan, q, k, v, ws=ws)
            assert e.value.status == 5 and "forced launch failure" in str(e.value)
            torch.cuda.synchronize()
            out = H.layer(plan, q, k, v, ws=ws)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    finally:
        H.debug_fail_launch(0)


def _guarded(nbytes, guard=4096, fill=0xA5):
    buf = torch.full((nbytes + 2 * guard,), fill, dtype=torch.uint8, device="cuda")
    return buf, buf[guard:guard + nbytes]


@pytest.mark.parametrize("partition", [0, 1, 2])
def test_workspace_index_and_output_canaries(partition):
    """Guard bytes before and after the workspace, the index buffer and the
    output stay untouched by a layer, a cached layer and the unmerged
    attention (every kernel writes inside the buffers it is given); the
    inputs are unchanged."""
    w = small_bf16(frames=6, heads=3, partition=partition)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    copies = [t.clone() for t in (q, k, v)]
    G = 4096
    wsb, ws = _guarded(plan.workspace_bytes, G)
    ixb, ix = _guarded(plan.index_bytes, G)
    n_out = q.numel() * 2
    outb, outs = _guarded(n_out, G)
    out = outs.view(torch.bfloat16).view(q.shape)
    idx = H.CachedIndex.__new__(H.CachedIndex)
    idx.buf = ix
    idx.c = H.Index(0, ix.data_ptr(), ix.numel(), 0)
    H.layer(plan, q, k, v, ws=ws, out=out, index=idx)
    H.layer_cached(plan, idx, q, k, v, ws=ws, out=out)
    dwb, dws = _guarded(plan.dense_workspace_bytes, G)
    H.attention_dense(plan, q, k, v, ws=dws, out=out)
    torch.cuda.synchronize()
    for name, b in (("workspace", wsb), ("index", ixb), ("output", outb), ("dense workspace", dwb)):
        assert bool((b[:G] == 0xA5).all()) and bool((b[-G:] == 0xA5).all()), name
    for a, c in zip((q, k, v), copies):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
