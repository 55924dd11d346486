"""CPU checks of the staged checker's block-local stages: the oracle's own
intermediates, laid out as an implementation hands them over, pass; a planted
mistake in any stage (a wrong match, a swapped selection, a member moved to
another group, one ulp on a deviation, one flipped outlier bit, one token
moved to another final slot) is caught."""
import numpy as np
import pytest

import gen
import oracle as O
from oracle import staged


def _case():
    w = gen.Workload(name="blk_chk", cfg_id=14, dtype="f32", heads=2, d_head=64, frames=4, grid_h=5, grid_w=6,
                     n_special=1, n_s=10, n_t=2, q_ratio=0.6, kv_ratio=0.5, outlier_pct=10.0)
    x = gen.layer_inputs(w)
    return w, x, O.Params.from_workload(w)


def _stream_items(x, p, ratio, stride):
    """Block-relative matches and scores (sources by block, then position) and
    the group label of every token, from the oracle."""
    s = O.dst_stride(ratio, stride)
    match, score = [], []
    for b in O.blocks(p):
        dpos, spos, mpos, sc = O.match_block(x[b.tokens], s)
        match.append(np.searchsorted(dpos, mpos))
        score.append(sc)
    m = O.match_stream(x, p, ratio, stride)
    return np.concatenate(match).astype(np.int32), np.concatenate(score).astype(np.float32), m.rep


def _fake_gpu(x, p):
    h = x["q"].shape[0]
    gpu = {k: [] for k in ("q_match", "q_score", "q_group", "kv_match", "kv_score", "kv_group")}
    for i in range(h):
        for t, ratio, stride, pre in (("q", p.q_ratio, p.q_dst_stride, "q"), ("k", p.kv_ratio, p.kv_dst_stride, "kv")):
            m, sc, rep = _stream_items(x[t][i], p, ratio, stride)
            gpu[pre + "_match"].append(m)
            gpu[pre + "_score"].append(sc)
            gpu[pre + "_group"].append(rep)
    gpu = {k: np.stack(v) for k, v in gpu.items()}
    delta = O.deviations(x["q"], list(gpu["q_group"]))
    mask = O.select_outliers(delta, O.outlier_budget(p))
    gpu["delta"] = delta
    gpu["outlier"] = mask.astype(np.uint8)
    gpu["q_slot"] = np.stack([O.restore_partition(gpu["q_group"][i], mask[i]) for i in range(h)])
    return gpu


def _check(x, p, gpu, out):
    return staged.check_layer(x["q"], x["k"], x["v"], p, gpu, out, out_tol=1e-6)


def test_oracle_intermediates_pass():
    w, x, p = _case()
    gpu = _fake_gpu(x, p)
    tr = O.layer(x["q"], x["k"], x["v"], p)
    rep = _check(x, p, gpu, tr.out)
    assert rep.n_src > 0 and rep.match_near_ties == 0 and rep.select_near_ties == 0 and rep.delta_nonexact == 0


def _first_block_sources(p, ratio):
    """(block, |S|, r, first source index of the block) of the first block with 0 < r < |S|."""
    s = O.dst_stride(ratio)
    k0 = 0
    for b in O.blocks(p):
        ns = b.n - (-(-b.n // s))
        r = O.merge_count(ratio, b.n, ns)
        if 0 < r < ns:
            return b, ns, r, k0
        k0 += ns
    raise AssertionError("no block with a proper selection")


@pytest.mark.parametrize("what", ["match", "selection", "member", "delta_ulp", "mask_bit", "slot"])
def test_planted_mistakes_are_caught(what):
    w, x, p = _case()
    gpu = _fake_gpu(x, p)
    tr = O.layer(x["q"], x["k"], x["v"], p)
    N = p.n_tokens
    if what == "match":  # a key source matched to its least similar destination
        b, ns, r, k0 = _first_block_sources(p, p.kv_ratio)
        dpos, spos, sim = O.block_similarity(x["k"][0][b.tokens], O.dst_stride(p.kv_ratio))
        i = int(np.argmax(sim.max(1) - sim.min(1)))
        gpu["kv_match"][0, k0 + i] = int(np.argmin(sim[i]))
    elif what == "selection":  # a merged key source swapped with an unmerged one, far from the r-th score
        b, ns, r, k0 = _first_block_sources(p, p.kv_ratio)
        s = O.dst_stride(p.kv_ratio)
        dpos, spos, sim = O.block_similarity(x["k"][0][b.tokens], s)
        so = sim.max(1)
        order = np.argsort(-so, kind="stable")
        best, worst = int(order[0]), int(order[-1])  # selected / not selected
        g = gpu["kv_group"][0].copy()
        tb, tw = b.tokens[spos[best]], b.tokens[spos[worst]]
        g[tb] = N + 1  # the best source leaves its group ...
        g[tw] = g[b.tokens[dpos[int(np.argmax(sim[worst]))]]]  # ... and the worst joins its match
        gpu["kv_group"] = np.stack([g, gpu["kv_group"][1]])
    elif what == "member":  # a merged query source moved to another destination's group
        q0 = gpu["q_group"][0].copy()
        sizes = np.bincount(np.unique(q0, return_inverse=True)[1])
        big = np.unique(q0)[sizes >= 2]
        a, c = big[0], big[1]
        mover = int(np.flatnonzero(q0 == a)[-1])
        q0[mover] = c
        gpu["q_group"] = np.stack([q0, gpu["q_group"][1]])
    elif what == "delta_ulp":  # one ulp on one deviation
        n = int(np.flatnonzero(gpu["delta"][1] > 0)[0])
        gpu["delta"][1, n] = np.nextafter(gpu["delta"][1, n], np.float32(np.inf))
    elif what == "mask_bit":  # one outlier bit flipped
        n = int(np.flatnonzero(gpu["outlier"][0])[0])
        gpu["outlier"][0, n] = 0
    elif what == "slot":  # one token moved to another final query slot
        fs = gpu["q_slot"][1].copy()
        u = np.unique(fs)
        n = int(np.flatnonzero(fs == u[3])[0])
        fs[n] = u[4]
        gpu["q_slot"] = np.stack([gpu["q_slot"][0], fs])
    with pytest.raises(staged.ParityError):
        _check(x, p, gpu, tr.out)
