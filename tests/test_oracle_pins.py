"""Pins of the CPU oracle against things other than itself.

Each check ties the oracle to what the method's pages and mathematics fix:

* hand-worked block with exact closed forms (tests/golden/hand_example.json);
* merge ratio 0 gives exact attention, checked against torch's
  scaled_dot_product_attention in fp64 (a library routine);
* outlier budget 100 % leaves every query unmerged;
* brute force on tiny blocks: double-loop cosine similarity, per-source
  argmax, exhaustive top-r over all subsets with exact rational sums, and a
  full sort for the global outlier choice;
* invariants: means are fp64 means of their members, unmerge copies,
  V follows K, block sizes n_b = n_s * n_t, head independence, block
  locality, nesting of outlier sets, zero deviation for unmerged tokens,
  token counts.

The absolute outputs of the full layer at the VGGT-shaped sizes are pinned
only through these properties: "parity unpinned" for those absolute values.
"""
import ast
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import gen
import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- helpers
def _expr(s: str) -> float:
    """Evaluate a closed form made of numbers, + - * / and sqrt()."""

    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant):
            return float(node.value)
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            return {ast.Add: a + b, ast.Sub: a - b, ast.Mult: a * b, ast.Div: a / b}[type(node.op)]
        if isinstance(node, ast.Call) and getattr(node.func, "id", "") == "sqrt":
            return math.sqrt(ev(node.args[0]))
        raise ValueError(s)

    return ev(ast.parse(s, mode="eval"))


def _hand():
    with open(os.path.join(HERE, "golden", "hand_example.json")) as f:
        ex = json.load(f)
    p = O.Params(**ex["params"])
    q = np.array(ex["q"], np.float32)[None]
    k = np.array(ex["k"], np.float32)[None]
    v = np.array(ex["v"], np.float32)[None]
    return ex, p, q, k, v


def _groups(rep):
    g = {}
    for n, r in enumerate(rep):
        g.setdefault(int(r), []).append(n)
    return sorted(g.values())


def _sdpa64(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q)[None], t(k)[None], t(v)[None], scale=scale)[0].numpy()


def _small(heads=2, frames=6, gh=5, gw=6, sp=2, n_s=8, n_t=3, qr=0.5, kr=0.5, pct=10.0, **kw):
    return O.Params(heads=heads, d_head=8, frames=frames, grid_h=gh, grid_w=gw, n_special=sp,
                    n_s=n_s, n_t=n_t, q_ratio=qr, kv_ratio=kr, outlier_pct=pct, **kw)


def _rand_qkv(p, seed=0, redundant=True):
    rng = np.random.default_rng(seed)
    N, d = p.n_tokens, p.d_head
    if redundant:
        base = rng.standard_normal((p.heads, 1, p.grid_h * p.grid_w, d))
        x = base + 0.3 * rng.standard_normal((p.heads, p.frames, p.grid_h * p.grid_w, d))
        full = np.empty((3, p.heads, p.frames, p.tokens_per_frame, d))
        for i in range(3):
            full[i, :, :, :p.n_special] = rng.standard_normal((p.heads, p.frames, p.n_special, d))
            full[i, :, :, p.n_special:] = x + 0.2 * rng.standard_normal(x.shape)
        full = full.reshape(3, p.heads, N, d)
    else:
        full = rng.standard_normal((3, p.heads, N, d))
    return [a.astype(np.float32) for a in full]


# ---------------------------------------------------------------- hand example
def test_hand_example_blocks_and_matches():
    ex, p, q, k, v = _hand()
    e = ex["expected"]
    bl = O.blocks(p)
    assert len(bl) == 1 and bl[0].n == e["n_b"] == p.n_s * p.n_t
    assert bl[0].tokens.tolist() == e["block_order_tokens"]
    assert O.dst_stride(p.q_ratio) == e["dst_stride"]
    m = O.match_stream(q[0], p, p.q_ratio, 0)
    for s, d in e["match"].items():
        assert m.match_dst[int(s)] == d
    for s, val in e["score"].items():
        assert abs(float(m.score[int(s)]) - _expr(val)) < 1e-6
    assert sorted(np.flatnonzero(m.selected).tolist()) == e["selected"]
    assert O.merge_count(p.q_ratio, 8, 6) == e["r"]
    assert _groups(m.rep) == e["groups"]


def test_hand_example_means_deviation_outliers():
    ex, p, q, k, v = _hand()
    e = ex["expected"]
    m = O.match_stream(q[0], p, p.q_ratio, 0)
    part = O.partition(m.rep)
    means = O.group_means(q[0], part)
    for rep, vals in e["q_means"].items():
        gi = int(np.flatnonzero(part.reps == int(rep))[0])
        assert np.allclose(means[gi], [_expr(x) for x in vals], atol=1e-6)
    km = O.match_stream(k[0], p, p.kv_ratio, 0)
    kp = O.partition(km.rep)
    vmeans = O.group_means(v[0], kp)  # V follows K's groups
    for rep, vals in e["v_means"].items():
        gi = int(np.flatnonzero(kp.reps == int(rep))[0])
        assert np.allclose(vmeans[gi], [_expr(x) for x in vals], atol=1e-6)
    delta = O.deviation(q[0], part, means)
    assert np.allclose(delta, [_expr(x) for x in e["delta"]], atol=1e-6)
    assert delta[3] == 0.0 and delta[7] == 0.0
    assert O.outlier_budget(p) == e["p25"]["k_o"]
    mo = O.select_outliers(delta[None], O.outlier_budget(p))
    assert np.flatnonzero(mo[0]).tolist() == e["p25"]["outliers"]
    fin = O.restore_partition(m.rep, mo[0])
    assert _groups(fin) == e["p25"]["final_groups"]
    assert len(set(fin.tolist())) == e["p25"]["L_q"]
    fp = O.partition(fin)
    fq = O.group_means(q[0], fp)
    for rep, vals in e["p25"]["final_q"].items():
        gi = int(np.flatnonzero(fp.reps == int(rep))[0])
        assert np.allclose(fq[gi], [_expr(x) for x in vals], atol=1e-6)


def test_hand_example_layer_output_vs_sdpa():
    """Whole layer on the hand block equals SDPA on the hand-derived merged rows."""
    ex, p, q, k, v = _hand()
    e = ex["expected"]
    tr = O.layer(q, k, v, p)
    fq = e["p25"]["final_q"]
    slots = sorted(int(r) for r in fq)
    Q = np.array([[_expr(x) for x in fq[str(r)]] for r in slots])
    kreps = sorted(int(r) for r in e["v_means"])
    K = np.array([[_expr(x) for x in e["q_means"][str(r)]] for r in kreps])  # k == q here
    V = np.array([[_expr(x) for x in e["v_means"][str(r)]] for r in kreps])
    o = _sdpa64(Q, K, V, 1.0)
    slot_of = {}
    for gi, grp in enumerate(e["p25"]["final_groups"]):
        for n in grp:
            slot_of[n] = slots.index(min(grp))
    want = np.stack([o[slot_of[n]] for n in range(8)])
    assert np.allclose(tr.out[0], want, atol=1e-6)
    # p = 100: every query is its own slot
    p100 = O.Params(**{**ex["params"], "outlier_pct": 100.0})
    assert O.outlier_budget(p100) == e["p100"]["k_o"]
    tr100 = O.layer(q, k, v, p100)
    assert len(set(tr100.q_final_rep[0].tolist())) == e["p100"]["L_q"]


# ---------------------------------------------------------------- limits (spec checks)
@pytest.mark.parametrize("sp", [0, 2])
def test_ratio_zero_is_exact_attention(sp):
    p = _small(sp=sp, qr=0.0, kr=0.0, pct=10.0)
    q, k, v = _rand_qkv(p, 1)
    tr = O.layer(q, k, v, p)
    for h in range(p.heads):
        ref = _sdpa64(q[h], k[h], v[h], p.scale)
        assert np.abs(tr.out[h] - ref).max() < 1e-5
        assert len(set(tr.q_final_rep[h].tolist())) == p.n_tokens
        assert len(set(tr.k_rep[h].tolist())) == p.n_tokens


def test_outlier_100_gives_unmerged_queries():
    p = _small(pct=100.0, qr=0.6, kr=0.5)
    q, k, v = _rand_qkv(p, 2)
    tr = O.layer(q, k, v, p)
    assert tr.outlier.all()
    for h in range(p.heads):
        assert np.array_equal(tr.q_final_rep[h], np.arange(p.n_tokens))
        kp = O.partition(tr.k_rep[h])
        kt, vt = O.group_means(k[h], kp), O.group_means(v[h], kp)
        ref = _sdpa64(q[h], kt, vt, p.scale)
        assert np.abs(tr.out[h] - ref).max() < 1e-5


def test_duplicate_queries_merge_exactly():
    """Q-only merge of exactly duplicated queries equals exact attention."""
    p = _small(heads=1, sp=0, qr=0.75, kr=0.0, pct=0.0, n_s=8, n_t=3)
    q, k, v = _rand_qkv(p, 3, redundant=False)
    # make every source an exact copy of the destination that starts its stride group
    for b in O.blocks(p):
        for i, tok in enumerate(b.tokens):
            q[0, tok] = q[0, b.tokens[(i // 4) * 4]]
    tr = O.layer(q, k, v, p)
    ref = _sdpa64(q[0], k[0], v[0], p.scale)
    assert np.abs(tr.out[0] - ref).max() < 1e-6
    assert len(set(tr.q_final_rep[0].tolist())) == sum(-(-b.n // 4) for b in O.blocks(p))


# ---------------------------------------------------------------- brute force
def _brute_block(xb, s, ratio):
    n = len(xb)
    dpos = [i for i in range(n) if i % s == 0]
    spos = [i for i in range(n) if i % s != 0]
    nrm = [math.sqrt(sum(float(c) * float(c) for c in row)) for row in xb]

    def cos(i, j):
        dot = sum(float(a) * float(b) for a, b in zip(xb[i], xb[j]))
        return dot / (max(nrm[i], 1e-12) * max(nrm[j], 1e-12))

    match, score = {}, {}
    for i in spos:
        best, bj = None, None
        for j in dpos:
            c = cos(i, j)
            if best is None or c > best:
                best, bj = c, j
        match[i], score[i] = bj, best
    r = min(len(spos), int(math.floor(ratio * n + 1e-9)))
    best_set, best_sum = None, None
    for sub in itertools.combinations(spos, r):  # lexicographic order of position tuples
        tot = sum(Fraction(score[i]) for i in sub)
        if best_sum is None or tot > best_sum:
            best_set, best_sum = sub, tot
    return match, score, set(best_set)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_blocks(seed):
    rng = np.random.default_rng(100 + seed)
    p = O.Params(heads=1, d_head=3, frames=3, grid_h=1, grid_w=4, n_special=0,
                 n_s=4, n_t=3, q_ratio=[0.25, 0.5, 0.6][seed % 3], kv_ratio=0.5,
                 outlier_pct=30.0)
    x = rng.standard_normal((p.n_tokens, p.d_head)).astype(np.float32)
    m = O.match_stream(x, p, p.q_ratio, 0)
    s = O.dst_stride(p.q_ratio)
    for b in O.blocks(p):
        xb = x[b.tokens]
        match, score, sel = _brute_block(xb, s, p.q_ratio)
        for i, j in match.items():
            assert m.match_dst[b.tokens[i]] == b.tokens[j]
            assert abs(m.score[b.tokens[i]] - score[i]) < 1e-6
        got = {i for i in range(b.n) if m.selected[b.tokens[i]]}
        assert got == sel


def test_brute_force_outlier_sort():
    rng = np.random.default_rng(7)
    delta = rng.random((3, 17)).astype(np.float32)
    delta[0, 3] = delta[2, 5] = delta[1, 1]  # exact ties: lower flat index first
    delta[:, :2] = 0.0
    for k_o in [0, 1, 5, 17, 30, 51]:
        flat = [(float(delta[h, n]), h * 17 + n) for h in range(3) for n in range(17)]
        pick = sorted(flat, key=lambda t: (-t[0], t[1]))[:k_o]
        want = np.zeros(51, bool)
        want[[i for _, i in pick]] = True
        assert np.array_equal(O.select_outliers(delta, k_o).reshape(-1), want)


# ---------------------------------------------------------------- invariants
def test_means_are_fp64_means_and_v_follows_k():
    p = _small()
    q, k, v = _rand_qkv(p, 4)
    tr = O.layer(q, k, v, p)
    for h in range(p.heads):
        for x, rep in [(q[h], tr.q_match[h].rep), (k[h], tr.k_rep[h]), (v[h], tr.k_rep[h])]:
            part = O.partition(rep)
            mu = O.group_means(x, part)
            for gi in range(len(part.reps)):
                mem = part.members[part.starts[gi]:part.starts[gi + 1]]
                assert np.abs(mu[gi] - x[mem].astype(np.float64).mean(0)).max() < 1e-6


def test_unmerge_copies_and_rows_come_from_o():
    p = _small(pct=20.0)
    q, k, v = _rand_qkv(p, 5)
    tr = O.layer(q, k, v, p)
    for h in range(p.heads):
        fin = tr.q_final_rep[h]
        for g in _groups(fin):
            rows = tr.out[h][g]
            assert (rows == rows[0]).all()


def test_blocks_partition_patch_tokens_and_sizes():
    for name in ["tiny", "vggt30", "vggt100", "vggt200", "vggt500"]:
        w = gen.WORKLOADS[name]
        p = O.Params.from_workload(w)
        pi = O.reorder_permutation(p)
        patch = np.flatnonzero(~O.is_special(p))
        assert np.array_equal(np.sort(pi), patch)
        for b in O.blocks(p):
            assert b.n == b.nf * b.run
            if b.nf == p.n_t and b.run == p.n_s:
                assert b.n == p.n_s * p.n_t
    inv = lambda name: sorted(
        (lambda c: [(n, c.count(n)) for n in set(c)])([b.n for b in O.blocks(O.Params.from_workload(gen.WORKLOADS[name]))]))
    assert inv("vggt30") == [(2670, 1), (3840, 10)]
    assert inv("vggt100") == [(890, 1), (1280, 10), (2670, 3), (3840, 30)]
    assert inv("vggt500") == [(1780, 1), (2560, 10), (2670, 16), (3840, 160)]
    assert O.blocks(O.Params.from_workload(gen.WORKLOADS["vggt30"]))[0].n == 128 * 30 == 3840


def test_token_counts_vggt30():
    """L_k, G_q and k_o at the 30-frame VGGT shape follow from the block table."""
    p = O.Params.from_workload(gen.WORKLOADS["vggt30"])
    bl = O.blocks(p)
    sq, sk = O.dst_stride(p.q_ratio), O.dst_stride(p.kv_ratio)
    assert (sq, sk) == (10, 4)
    Lk = sum(b.n - O.merge_count(p.kv_ratio, b.n, b.n - (-(-b.n // sk))) for b in bl) + p.frames * p.n_special
    Gq = sum(b.n - O.merge_count(p.q_ratio, b.n, b.n - (-(-b.n // sq))) for b in bl) + p.frames * p.n_special
    assert (Lk, Gq, O.outlier_budget(p)) == (20685, 4257, 65952)


def test_head_independence_and_block_locality():
    p = _small(heads=3, pct=0.0)
    q, k, v = _rand_qkv(p, 6)
    tr = O.layer(q, k, v, p)
    perm = [2, 0, 1]
    tr2 = O.layer(q[perm], k[perm], v[perm], p)
    for i, h in enumerate(perm):
        assert np.array_equal(tr2.q_match[i].rep, tr.q_match[h].rep)
        assert np.allclose(tr2.out[i], tr.out[h], atol=1e-12)
    # perturb everything outside block 0 of head 0: block 0's matches stay
    b0 = O.blocks(p)[0].tokens
    q2 = q.copy()
    mask = np.ones(p.n_tokens, bool)
    mask[b0] = False
    q2[0, mask] += np.random.default_rng(1).standard_normal((mask.sum(), p.d_head)).astype(np.float32)
    m1 = O.match_stream(q[0], p, p.q_ratio, 0)
    m2 = O.match_stream(q2[0], p, p.q_ratio, 0)
    assert np.array_equal(m1.rep[b0], m2.rep[b0]) and np.array_equal(m1.selected[b0], m2.selected[b0])
    # perturbing head 1 leaves head 0's matching untouched
    q3 = q.copy()
    q3[1] += 1.0
    assert np.array_equal(O.match_stream(q3[0], p, p.q_ratio, 0).rep, m1.rep)


def test_outlier_nesting_and_unmerged_zero():
    p = _small(heads=3)
    q, k, v = _rand_qkv(p, 8)
    reps = [O.match_stream(q[h], p, p.q_ratio, 0).rep for h in range(p.heads)]
    delta = O.deviations(q, reps)
    spec = O.is_special(p)
    for h in range(p.heads):
        sizes = np.bincount(np.unique(reps[h], return_inverse=True)[1])
        single = sizes[np.unique(reps[h], return_inverse=True)[1]] == 1
        assert (delta[h][spec] == 0).all() and (delta[h][single] == 0).all()
    prev = None
    for pct in [0, 5, 10, 20, 50, 100]:
        m = O.select_outliers(delta, int(pct * delta.size // 100))
        if prev is not None:
            assert (m | ~prev).all() or (prev <= m).all()
            assert (prev & ~m).sum() == 0
        prev = m


def test_specials_stay_unmerged_and_counts():
    p = _small(sp=3, qr=0.75, kr=0.5)
    q, k, v = _rand_qkv(p, 9)
    tr = O.layer(q, k, v, p)
    spec = np.flatnonzero(O.is_special(p))
    for h in range(p.heads):
        for rep in [tr.q_match[h].rep, tr.k_rep[h], tr.q_final_rep[h]]:
            groups = {}
            for n, r in enumerate(rep):
                groups.setdefault(r, []).append(n)
            for s in spec:
                assert groups[rep[s]] == [s]
        # L_k = sum over blocks (n - r) + specials
        sk = O.dst_stride(p.kv_ratio)
        Lk = sum(b.n - O.merge_count(p.kv_ratio, b.n, b.n - (-(-b.n // sk))) for b in O.blocks(p)) + len(spec)
        assert len(set(tr.k_rep[h].tolist())) == Lk


def test_generator_shapes_and_bf16():
    w = gen.WORKLOADS["tiny"]
    x = gen.layer_inputs(w)
    assert x["q"].shape == (1, 1024, 64) and x["q"].dtype == np.float32
    w1 = gen.WORKLOADS["vggt30"].with_(frames=2)
    y = gen.layer_inputs(w1, heads=[0, 5])
    assert y["k"].shape == (2, 2 * 1374, 64)
    assert np.array_equal(gen.round_bf16(y["v"]), y["v"])  # bf16 representable
    # regenerating one head alone gives the same bytes
    z = gen.layer_inputs(w1, heads=[5])
    assert np.array_equal(z["q"][0], y["q"][1])
    # round-to-nearest-even on an exact half-way case
    a = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], np.float32)
    assert gen.round_bf16(a).tolist() == [1.0, 1.0 + 2 ** -6]
