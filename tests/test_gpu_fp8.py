"""FP8 (OCP e4m3) attention scores on the GPU against the oracle.

The oracle defines the variant exactly (e4m3 rounding, power-of-two scales
per query row and per head's keys, exact products; readings R41-R44), so the
GPU output differs from it only by the fp32 sums and the bf16 probabilities,
as the bf16 path does from its oracle: the same 2e-2 x RMS bar applies.  The
key and query codes are compared bit for bit where the oracle's merged rows
equal the stored ones (no outliers restored), and the merge indices are the
bf16 layer's (FP8 enters only the scores).
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


def small_fp8(frames=6, heads=4, n_t=3, **kw):
    return gen.WORKLOADS["vggt30"].with_(name="small_fp8", cfg_id=7, frames=frames, heads=heads, n_t=n_t,
                                         attn_fp8=True, **kw)


def _e4m3(codes: np.ndarray) -> np.ndarray:
    """Values of e4m3 bytes (torch's float8_e4m3fn decoding)."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


@pytest.mark.parametrize("seed", [gen.DEFAULT_SEED, gen.DEFAULT_SEED + 1])
def test_fp8_small_layer_full_outputs(seed):
    w = small_fp8()
    x = gen.layer_inputs(w, seed=seed)
    p = O.Params.from_workload(w)
    assert p.attn_fp8
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    say(f"[fp8 small seed {seed}] q rows per head {np.diff(gpu['cu_q']).tolist()}")
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    say("  ", rep.as_dict())
    # the bf16 layer on the same inputs: same partitions, different scores
    w16 = w.with_(attn_fp8=False)
    _, _, _, out16, gpu16, _ = run_layer(w16, x)
    for it in ("q_slot", "kv_group", "cu_q", "outlier"):
        assert np.array_equal(gpu[it], gpu16[it]), it
    rel = np.sqrt(((out - out16) ** 2).mean()) / np.sqrt((out16 ** 2).mean())
    say(f"   fp8 vs bf16 layer output: relative RMS difference {rel:.3g}")
    assert 0 < rel < 0.1


def test_fp8_operands_are_the_oracle_codes():
    """No outliers: every merged query row is the plain mean of its group, so
    the stored bf16 operands equal the oracle's and every e4m3 code and
    exponent of the score product must match the oracle's quantisation."""
    w = small_fp8(outlier_pct=0.0)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x)
    staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    gpu.update({it: H.debug_read(plan, ws, it) for it in H.FP8_ITEMS})
    h = w.heads
    lk, lkp = plan.info["kv_len"], -(-plan.info["kv_len"] // 64) * 64
    k8 = _e4m3(gpu["k8"]).reshape(h, lkp, 64)
    q8 = _e4m3(gpu["q8"]).reshape(-1, 64)
    cu = gpu["cu_q"]
    tr = O.layer(x["q"], x["k"], x["v"], p)
    for i in range(h):
        qp, kp = O.partition(tr.q_final_rep[i]), O.partition(tr.k_rep[i])
        qm, km, vm = O.group_means(x["q"][i], qp), O.group_means(x["k"][i], kp), O.group_means(x["v"][i], kp)
        qb, kb, _ = O.fp8_operands(qm, km, vm, p.scale)
        k8o, eko = O.fp8_quantize(kb, per_row=False)
        q8o, eqo = O.fp8_quantize(qb, per_row=True)
        assert int(gpu["kexp"][i]) == int(eko), f"head {i}: key exponent"
        # GPU key slot s against the oracle's slot of the same group (its first token)
        _, first = np.unique(gpu["kv_group"][i], return_index=True)
        got_k = k8[i, :lk]
        ref_k = k8o[kp.group_of[first]]
        nk = int((got_k != ref_k).sum())
        assert nk == 0, f"head {i}: {nk} key codes differ"
        assert (k8[i, lk:] == 0).all()
        # queries: the packed row of every token against the oracle's row of its group
        slot = gpu["q_slot"][i]
        got_q = q8[slot]
        ref_q = q8o[qp.group_of]
        nq = int((got_q != ref_q).any(axis=1).sum())
        assert nq == 0, f"head {i}: {nq} tokens read query codes that differ"
        assert np.array_equal(gpu["qexp"][slot], eqo[qp.group_of]), f"head {i}: query exponents"
    say(f"[fp8 codes] keys {lk} x {h} heads, query rows {cu[-1]}: all equal")


@pytest.mark.parametrize("split", [1, 8])
def test_fp8_key_splits_and_tail_tiles(split):
    """1 or 8 key splits (8 gives tail tiles 16 splits) on a layer with several
    query tiles per head and partly filled rounds, every output row."""
    w = small_fp8(frames=8, heads=16)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, x, attn_split=split)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, rel_tol=BF16_REL)
    say(f"[fp8 split {split}]", rep.as_dict())


def _orthogonal_offset(x, big=600.0):
    """Keys in channels 0-31, queries with a large constant in channels 32-63:
    the norm bound exceeds every score by far more than 60 (log2 units), so
    every unit takes the exact (running-max) path."""
    q = x["q"].copy()
    k = x["k"].copy()
    k[..., 32:] = 0.0
    q[..., 32:] = big
    return {"q": gen.round_bf16(q), "k": gen.round_bf16(k), "v": x["v"]}


def test_fp8_fallback_exact_path():
    w = small_fp8(frames=4, heads=2)
    xs = _orthogonal_offset(gen.layer_inputs(w))
    p = O.Params.from_workload(w)
    plan, ws, dev, out, gpu, _ = run_layer(w, xs)
    fb = int(gpu["attn_fallback"][0])
    say(f"[fp8 fallback] units recomputed exactly: {fb}")
    assert fb > 0
    rep = staged.check_layer(xs["q"], xs["k"], xs["v"], p, gpu, out, rel_tol=BF16_REL)
    say("  ", rep.as_dict())


def test_fp8_cached_layer_and_shared_index():
    """Cached layers with FP8 scores against the oracle, on an index filled by
    the FP8 layer, and the same index exported and imported into a bf16 plan
    (merge indices do not depend on the score type)."""
    w = small_fp8(frames=6, heads=4)
    x0 = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out0, gpu, idx = run_layer(w, x0, keep_index=True)
    staged.check_layer(x0["q"], x0["k"], x0["v"], p, gpu, out0, rel_tol=BF16_REL)
    qf = [staged.canonical(gpu["q_slot"][h]) for h in range(w.heads)]
    kr = [staged.canonical(gpu["kv_group"][h]) for h in range(w.heads)]
    x1 = gen.layer_inputs(w, layer=1)
    q, k, v = (to_dev(x1[t], w.dtype) for t in "qkv")
    out1 = H.layer_cached(plan, idx, q, k, v, ws=ws).float().cpu().numpy()
    ref1 = O.layer_cached(x1["q"], x1["k"], x1["v"], p, qf, kr)
    rms = np.sqrt((ref1 ** 2).mean())
    err = np.abs(out1 - ref1).max()
    say(f"[fp8 cached] err {err:.3g} rms {rms:.3g}")
    assert err <= BF16_REL * rms
    # the index in a bf16 plan: bf16 scores on the same partitions
    plan16 = H.Plan.from_workload(w.with_(attn_fp8=False))
    idx16 = H.index_import(plan16, H.index_export(plan, idx))
    ws16 = H.workspace(plan16)
    out16 = H.layer_cached(plan16, idx16, q, k, v, ws=ws16).float().cpu().numpy()
    ref16 = O.layer_cached(x1["q"], x1["k"], x1["v"], O.Params.from_workload(w.with_(attn_fp8=False)), qf, kr)
    assert np.abs(out16 - ref16).max() <= BF16_REL * np.sqrt((ref16 ** 2).mean())


@pytest.mark.timeout(900)
def test_fp8_vggt500_layer_and_cached_layer():
    """500 frames (687,000 tokens): the FP8 layer's index stages on every
    head, outputs on sampled rows (one per 256-row query tile) of the oracle
    heads, then one cached FP8 layer on layer-1 inputs of those heads."""
    w = gen.WORKLOADS["vggt500"].with_(attn_fp8=True)
    oh = gen.oracle_heads(w)
    say(f"[fp8 vggt500] N={w.n_tokens} oracle heads {oh}")
    x0 = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    plan, ws, dev, out0, gpu, idx = run_layer(w, x0, keep_index=True)
    tiles = [tile_rows(gpu["q_slot"][h], gpu["cu_q"], h) for h in oh]
    rows = np.unique(np.concatenate([sample_rows(w.n_tokens, 256, 3)] + tiles))
    say(f"   output rows checked per oracle head: {len(rows)}")
    rep = staged.check_layer(x0["q"], x0["k"], x0["v"], p, gpu, out0, out_heads=oh, rows=rows,
                             rel_tol=BF16_REL, workers=WORKERS)
    say("  ", rep.as_dict())
    qf = {h: staged.canonical(gpu["q_slot"][h]) for h in oh}
    kr = {h: staged.canonical(gpu["kv_group"][h]) for h in oh}
    q, k, v = dev
    del out0, gpu
    for l, xl in gen.layer_stack(w, heads=oh, layers=2):
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
            say(f"  cached layer {l} head {h}: err {err:.3g} rms {rms:.3g}")
            assert err <= BF16_REL * rms
