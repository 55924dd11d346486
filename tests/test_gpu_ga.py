"""GPU parity of the geometry-aware partition ("LiteVGGT: Boosting Vanilla
VGGT via Geometry-aware Cached Token Merging", key designs 1-3) against the
CPU oracle, staged like the block-local layer:

  variance map and token classes bit for bit; every source's destination is
  the oracle's most similar one or a counted near-tie (|dsim| < 1e-5), its
  cosine within 1e-5; groups exactly; deviations bit for bit on the GPU's
  groups; the outlier mask exactly; outputs within 1e-4 (fp32) or
  2e-2 * RMS (bf16).
"""
import numpy as np
import pytest
import torch

import gen
import oracle as O
from oracle import staged
import token_merged_global_amd as H

from gpu_util import BF16_REL, F32_ABS, read_all, run_layer, say, to_dev

pytestmark = pytest.mark.gpu


def ga(w, pct=10.0, **kw):
    return w.with_(partition=1, protect_pct=pct, **kw)


def small(frames=6, heads=4, **kw):
    return ga(gen.WORKLOADS["vggt30"].with_(name="small", cfg_id=7, frames=frames, heads=heads, n_t=3), **kw)


def _key_lengths(gpu, heads):
    """Keys per head from the library equal the number of key groups."""
    kl = gpu["kv_len"]
    want = [len(np.unique(gpu["kv_group"][h])) for h in range(heads)]
    assert list(kl) == want, (list(kl), want)
    return kl


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1])
def test_ga_tiny_fp32(seed):
    w = ga(gen.WORKLOADS["tiny"])
    say(f"[ga tiny fp32] seed={seed}")
    x = gen.layer_inputs(w, seed=seed)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    _key_lengths(gpu, w.heads)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, out_tol=F32_ABS)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
    if rep.match_near_ties == 0 and rep.outlier_threshold_ties == 0:
        tr = O.layer(x["q"], x["k"], x["v"], p)
        assert np.abs(out - tr.out).max() <= F32_ABS


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1])
def test_ga_small_bf16_full_outputs(seed):
    w = small()
    say(f"[ga small bf16] seed={seed} N={w.n_tokens}")
    x = gen.layer_inputs(w, seed=seed)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    kl = _key_lengths(gpu, w.heads)
    assert (kl <= plan.info["kv_len"]).all() and (kl < w.n_tokens).all()
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL, workers=4)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0


@pytest.mark.parametrize("gh,gw,sp,pct,dtype", [(5, 7, 2, 20.0, "bf16"), (9, 11, 1, 0.0, "bf16"),
                                                (7, 5, 3, 100.0, "bf16"), (6, 6, 0, 35.0, "f32")])
def test_ga_odd_grids_and_protect_shares(gh, gw, sp, pct, dtype):
    """Odd grid edges (clipped 2x2 cells and 3x3 windows), no protection,
    everything protected (every token its own group: exact attention) and
    key counts far below one attention tile per split."""
    w = gen.Workload(name="ga_odd", cfg_id=12, dtype=dtype, heads=3, d_head=64, frames=5, grid_h=gh, grid_w=gw,
                     n_special=sp, n_s=16, n_t=2, q_ratio=0.5, kv_ratio=0.5, outlier_pct=10.0, partition=1,
                     protect_pct=pct)
    say(f"[ga odd] grid {gh}x{gw} specials {sp} protect {pct} {dtype}")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    kl = _key_lengths(gpu, w.heads)
    kw = dict(rel_tol=BF16_REL) if dtype == "bf16" else dict(out_tol=F32_ABS)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, **kw)
    say("  ", rep.as_dict(), "keys per head", list(kl))
    assert rep.delta_nonexact == 0
    if pct == 100.0:
        assert (kl == w.n_tokens).all()
        for h in range(w.heads):
            ref = O.attention(x["q"][h], x["k"][h], x["v"][h], p.scale)
            tol = BF16_REL * np.sqrt((ref ** 2).mean()) if dtype == "bf16" else F32_ABS
            assert np.abs(out[h] - ref).max() <= tol


def test_ga_vggt30_layer():
    """30 frames x 1374 tokens, 16 heads: variance, classes, matches and
    groups of every head and stream; outputs on sampled rows."""
    w = ga(gen.WORKLOADS["vggt30"])
    say("[ga vggt30]")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    kl = _key_lengths(gpu, w.heads)
    rows = np.sort(np.random.default_rng(3).choice(w.n_tokens, 256, replace=False))
    rows = np.unique(np.r_[rows, [0, 1, 5, w.n_tokens - 1]])
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rows=rows, rel_tol=BF16_REL, workers=8)
    say("  ", rep.as_dict(), "keys per head", int(kl.min()), "-", int(kl.max()))
    assert rep.delta_nonexact == 0


def test_ga_repeat_runs_are_bit_identical():
    """Slot placement uses atomic counters; the member order, and so every
    output, must not depend on their order."""
    w = small(frames=5, heads=3)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    o1, i1 = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    o1 = o1.clone()
    d1 = {it: H.debug_read(plan, ws, it, index=i1) for it in H.debug_items(plan)}
    o2, i2 = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    d2 = {it: H.debug_read(plan, ws, it, index=i2) for it in H.debug_items(plan)}
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for it in d1:
        assert np.array_equal(d1[it], d2[it]), it
    # both indices drive identical cached layers (the index bytes past each
    # head's lengths are not written, so the raw buffers are not compared)
    c1 = H.layer_cached(plan, i1, q, k, v, ws=ws).clone()
    c2 = H.layer_cached(plan, i2, q, k, v, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


def test_ga_cached_layer_and_index_round_trip():
    """A cached layer reuses the geometry-aware groups (LiteVGGT page, key
    design 3), per-head key counts included, also through host memory."""
    w = small(frames=5, heads=2)
    x0 = gen.layer_inputs(w)
    x1 = {t: gen.round_bf16(x0[t] + np.random.default_rng(5).normal(0, 0.02, x0[t].shape).astype(np.float32))
          for t in "qkv"}
    p = O.Params.from_workload(w)
    plan = H.Plan.from_workload(w)
    dev0 = [to_dev(x0[t], w.dtype) for t in "qkv"]
    dev1 = [to_dev(x1[t], w.dtype) for t in "qkv"]
    ws = H.workspace(plan)
    _, idx = H.layer(plan, *dev0, ws=ws, keep_index=True)
    torch.cuda.synchronize()
    q_slot = H.debug_read(plan, ws, "q_slot", index=idx).reshape(w.heads, -1)
    kv_group = H.debug_read(plan, ws, "kv_group").reshape(w.heads, -1)
    out1 = H.layer_cached(plan, idx, *dev1, ws=ws).float().cpu().numpy()
    qf = [staged.canonical(q_slot[h]) for h in range(w.heads)]
    kr = [staged.canonical(kv_group[h]) for h in range(w.heads)]
    ref = O.layer_cached(x1["q"], x1["k"], x1["v"], p, qf, kr)
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(out1 - ref).max()
    say(f"[ga cached] err {err:.3g} rms {rms:.3g}")
    assert err <= BF16_REL * rms
    host = H.index_export(plan, idx)
    o2 = H.layer_cached(plan, H.index_import(plan, host), *dev1, ws=ws).float().cpu().numpy()
    assert np.array_equal(o2, out1)
    # the block-local plan of the same shape refuses this index
    blk = H.Plan.from_workload(w.with_(partition=0))
    if blk.index_bytes == plan.index_bytes:
        with pytest.raises(H.HttmError):
            H.index_import(blk, host)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ga_variance_map_tiny_values(dtype):
    """Inputs scaled by 2^-66: window sums of squares fall below 2^-125 (the
    subnormal range), where the variance kernel's fast quotient by 6 hands
    over to plain division; the map and the classes stay bit-exact."""
    w = gen.Workload(name="ga_tiny_vals", cfg_id=14, dtype=dtype, heads=2, d_head=64, frames=3, grid_h=7,
                     grid_w=9, n_special=1, n_s=16, n_t=2, q_ratio=0.5, kv_ratio=0.5, outlier_pct=10.0,
                     partition=1, protect_pct=10.0)
    x = gen.layer_inputs(w)
    xs = {t: (x[t] * np.float32(2.0 ** -66)).astype(np.float32) for t in "qkv"}
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, xs)
    var = gpu["ga_var"].reshape(2, w.heads, -1)
    role = gpu["ga_role"].reshape(2, w.heads, -1)
    tiny = 0
    for st, t in enumerate("qk"):
        for h in range(w.heads):
            want = O.token_variance_map(xs[t][h], p)
            assert np.array_equal(var[st, h], want), (t, h, np.flatnonzero(var[st, h] != want)[:5])
            assert np.array_equal(role[st, h], O.ga_roles(want, p)), (t, h)
            tiny += int(((want > 0) & (want < 2.0 ** -125)).sum())
    say(f"[ga tiny values {dtype}] variance entries below 2^-125: {tiny}")
    assert tiny > 0


def _index_regions(h, n, lk):
    """Byte offsets of the index regions (64-byte header, then each region
    at the next 256-byte boundary, in the layout order of the library)."""
    al = lambda x: (x + 255) & ~255
    sizes = [("header", 64), ("k_members", 4 * h * n), ("k_off", 4 * h * (lk + 1)), ("fmembers", 4 * h * n),
             ("foff", 4 * h * (n + 1)), ("slot", 4 * h * n), ("lenq", 4 * h), ("cu_q", 4 * (h + 1)),
             ("lenk", 4 * h)]
    off, cur = {}, 0
    for name, size in sizes:
        off[name] = cur
        cur = al(cur + size)
    return off, cur


def test_ga_index_import_checks_key_counts():
    """An imported geometry-aware index is checked on the host: the per-head
    key counts must lie in [1, kv_len] and the key offsets past them must be
    empty (equal to N)."""
    w = small(frames=4, heads=2)
    x = gen.layer_inputs(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    _, idx = H.layer(plan, q, k, v, ws=ws, keep_index=True)
    host = H.index_export(plan, idx)
    h, n, lk = w.heads, w.n_tokens, plan.info["kv_len"]
    off, total = _index_regions(h, n, lk)
    assert total == plan.index_bytes == host.nbytes
    lenk = host[off["lenk"]:off["lenk"] + 4 * h].view(np.int32)
    kl = H.debug_read(plan, ws, "kv_len", index=idx)
    assert np.array_equal(lenk, kl) and (kl < lk).all()
    ko = host[off["k_off"]:off["k_off"] + 4 * h * (lk + 1)].view(np.int32).reshape(h, lk + 1)
    assert (ko[0, kl[0]:] == n).all() and ko[0, 0] == 0
    H.index_import(plan, host)  # the untouched bytes pass
    for bad in (0, lk + 1):
        b = host.copy()
        b[off["lenk"]:off["lenk"] + 4].view(np.int32)[0] = bad
        with pytest.raises(H.HttmError) as e:
            H.index_import(plan, b)
        assert e.value.status == 4
    b = host.copy()
    b[off["k_off"]:off["k_off"] + 4 * h * (lk + 1)].view(np.int32).reshape(h, lk + 1)[1, kl[1] + 1] = n - 1
    with pytest.raises(H.HttmError) as e:
        H.index_import(plan, b)
    assert e.value.status == 4


@pytest.mark.parametrize("case", [dict(frames=1, grid_h=6, grid_w=7, n_special=1),
                                  dict(frames=6, grid_h=1, grid_w=1, n_special=2),
                                  dict(frames=3, grid_h=2, grid_w=9, n_special=0),
                                  dict(frames=2, grid_h=64, grid_w=64, n_special=1, dtype="bf16")])
def test_ga_edge_geometry(case):
    """One frame (no sources at all: exact attention), one patch per frame,
    a 2-row grid, the largest frame (64 x 64 patches, bf16): the
    geometry-aware layer against the oracle."""
    case = dict(case)
    dtype = case.pop("dtype", "f32")
    w = gen.Workload(name="ga_edge", cfg_id=22, dtype=dtype, heads=2, d_head=64, n_s=4, n_t=2, q_ratio=0.5,
                     kv_ratio=0.5, outlier_pct=10.0, partition=1, protect_pct=20.0, **case)
    say(f"[ga edge] {case}")
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    tol = dict(rel_tol=BF16_REL) if dtype == "bf16" else dict(out_tol=F32_ABS)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, workers=4, **tol)
    say("  ", rep.as_dict())
    assert rep.delta_nonexact == 0
    if case["frames"] == 1:
        assert rep.n_src == 0


def test_ga_match_timing_stage():
    """The global match has its own timing stage: recorded for every call
    under the geometry-aware partition, never under the block-local one,
    and inside the span of the whole partition (the similarity stage)."""
    say("[ga timing stage]")
    for part in (1, 0):
        w = small(frames=4).with_(partition=part)
        x = gen.layer_inputs(w, seed=gen.DEFAULT_SEED)
        plan = H.Plan.from_workload(w)
        q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
        ws = H.workspace(plan)
        H.set_timing(["sim", "ga_match"])
        try:
            for _ in range(3):
                H.layer(plan, q, k, v, ws=ws)
            torch.cuda.synchronize()
            st, calls = H.get_timing()
        finally:
            H.set_timing([])
        say("  ", part, calls, st["sim"], st["ga_match"])
        assert calls == 3
        assert st["sim"] > 0
        if part == 1:
            assert 0 < st["ga_match"] <= st["sim"]
        else:
            assert st["ga_match"] == 0


@pytest.mark.timeout(300)
def test_ga_constant_tokens_one_huge_group():
    """Every patch token of q and k the same row (per head): all cosines tie,
    every source joins the first destination, so one group holds every
    source (26,187 at 30 frames) and that destination.  The member lists come
    from a stable sort by slot, linear in N whatever the group sizes."""
    w = gen.WORKLOADS["vggt30"].with_(heads=2, partition=1, protect_pct=10.0)
    x = gen.layer_inputs(w)
    sp = np.arange(w.n_tokens) % w.tokens_per_frame < w.n_special
    for t in "qk":
        for h in range(w.heads):
            x[t][h][~sp] = x[t][h][w.n_special]
    p = O.Params.from_workload(w)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ws = H.workspace(plan)
    out = H.layer(plan, q, k, v, ws=ws)
    torch.cuda.synchronize()
    gpu = read_all(plan, ws, w.heads)
    sizes = np.bincount(gpu["kv_group"][0])
    n_src = int((gpu["ga_role"].reshape(2, w.heads, -1)[1, 0] == O.ROLE_SRC).sum())
    say(f"[ga constant] largest key group {sizes.max()} of {w.n_tokens} tokens ({n_src} sources)")
    assert sizes.max() == n_src + 1  # every source joins the first destination
    rows = np.unique(np.r_[np.random.default_rng(2).choice(w.n_tokens, 128, replace=False), 0, w.n_tokens - 1])
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out.float().cpu().numpy(), rows=rows,
                             rel_tol=BF16_REL, out_half_ulp=True, match_heads=[0])
    say("  ", rep.as_dict())
