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


# --------------------------------------------------------------------------
# Geometry-aware three-class partition (LiteVGGT page, key designs 1-3)
# --------------------------------------------------------------------------
def _ga_params(**kw):
    base = dict(heads=1, d_head=64, frames=2, grid_h=4, grid_w=5, n_special=1, n_s=4, n_t=2, q_ratio=0.5,
                kv_ratio=0.5, outlier_pct=0.0, partition=1, protect_pct=10.0)
    base.update(kw)
    return O.Params(**base)


def test_variance_map_closed_forms():
    """Constant field: v = 0.  Channel 0 = column index on a 4x5 grid: the 3x3
    window of an interior patch holds columns x-1..x+1 (variance 2/3), an edge
    or corner patch two columns (variance 1/4); v averages over the 64 channels."""
    p = _ga_params()
    T = p.tokens_per_frame
    x = np.ones((p.n_tokens, 64), np.float32)
    assert np.all(O.token_variance_map(x, p) == 0.0)
    x = np.zeros((p.n_tokens, 64), np.float32)
    cols = np.tile(np.arange(5, dtype=np.float32), 4)
    for f in range(p.frames):
        x[f * T + 1:(f + 1) * T, 0] = cols
    v = O.token_variance_map(x, p)
    for f in range(p.frames):
        vf = v[f * T + 1:(f + 1) * T].reshape(4, 5)
        assert v[f * T] == 0.0  # special token
        assert np.allclose(vf[:, 1:4], (2.0 / 3.0) / 64, rtol=1e-6)
        assert np.allclose(vf[:, [0, 4]], 0.25 / 64, rtol=1e-6)


@pytest.mark.parametrize("seed", [0, 1])
def test_variance_map_brute_force(seed):
    """Against explicit per-patch windows in fp64 (clipped 3x3 neighbourhoods)."""
    p = _ga_params(frames=2, grid_h=5, grid_w=6, n_special=2)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((p.n_tokens, 64)).astype(np.float32)
    v = O.token_variance_map(x, p)
    T, H_, W_ = p.tokens_per_frame, p.grid_h, p.grid_w
    for f in range(p.frames):
        for y in range(H_):
            for xx in range(W_):
                win = [x[f * T + p.n_special + yy * W_ + xc].astype(np.float64)
                       for yy in range(max(0, y - 1), min(H_, y + 2)) for xc in range(max(0, xx - 1), min(W_, xx + 2))]
                w = np.stack(win)
                ref = float(np.mean(w.var(axis=0)))
                assert abs(float(v[f * T + p.n_special + y * W_ + xx]) - ref) <= 1e-5 * max(1.0, ref)


def test_ga_roles_hand_example():
    """4x4 grid, 2 frames, 10 % protected (k = floor(1.6) = 1 per frame).
    Frame 0: the top patch is protected, the other 15 are destinations.
    Frame 1: top patch protected; each 2x2 cell's lowest unprotected patch is
    a destination (ties to the smaller index); the rest are sources."""
    p = _ga_params(frames=2, grid_h=4, grid_w=4, n_special=0)
    v = np.zeros(32, np.float32)
    v[:16] = np.arange(16, dtype=np.float32)  # frame 0: patch 15 is the top
    f1 = np.array([5, 1, 2, 9,
                   3, 7, 2, 2,
                   4, 4, 8, 6,
                   4, 0.5, 6, 10], np.float32)  # top: patch 15 (10); cells below
    v[16:] = f1
    role = O.ga_roles(v, p)
    S, D, P = O.ROLE_SRC, O.ROLE_DST, O.ROLE_PROTECT
    assert role[15] == P and np.all(role[:15] == D)
    want = np.full(16, S, np.int8)
    want[15] = P
    want[1] = D    # cell (0,0), patches {0, 1, 4, 5} with {5, 1, 3, 7} -> patch 1
    want[2] = D    # cell (0,1), patches {2, 3, 6, 7} with {2, 9, 2, 2} -> 2, 6, 7 tie -> patch 2
    want[13] = D   # cell (1,0), patches {8, 9, 12, 13} with {4, 4, 4, 0.5} -> patch 13
    want[11] = D   # cell (1,1), patches {10, 11, 14, 15} with {8, 6, 6, 10 (protected)} -> 11 and 14 tie -> 11
    assert role[16:].tolist() == want.tolist()


def test_ga_roles_full_cell_and_odd_edges():
    """A cell whose patches are all protected has no destination; on a 3x5
    grid the last row and column form clipped cells."""
    p = _ga_params(frames=2, grid_h=3, grid_w=5, n_special=0, protect_pct=27.0)  # k = floor(4.05) = 4
    v = np.zeros(30, np.float32)
    f1 = np.array([9, 9, 0, 1, 2,
                   9, 9, 3, 4, 5,
                   6, 7, 8, 0.5, 0.25], np.float32)  # top 4: patches 0, 1, 5, 6 (one full cell)
    v[15:] = f1
    role = O.ga_roles(v, p)[15:]
    assert [int(i) for i in np.flatnonzero(role == O.ROLE_PROTECT)] == [0, 1, 5, 6]
    # cells: (0,0) all protected; (0,1) {0, 1, 3, 4} -> 2; (0,2) {2, 5} -> 4; (1,0) {6, 7} -> 10;
    # (1,1) {8, 0.5} -> 13; (1,2) {0.25} -> 14
    assert [int(i) for i in np.flatnonzero(role == O.ROLE_DST)] == [2, 4, 10, 13, 14]


@pytest.mark.parametrize("seed", [0, 1])
def test_ga_match_brute_force(seed):
    """Every source joins its most similar destination over the whole
    sequence (fp64 brute force); groups: destination + its sources, protected
    and special tokens alone."""
    p = _ga_params(frames=3, grid_h=4, grid_w=6, n_special=1, protect_pct=20.0)
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((p.n_tokens, 64)).astype(np.float32)
    m = O.ga_match_stream(x, p)
    role = O.ga_roles(O.token_variance_map(x, p), p)
    src, dst = np.flatnonzero(role == O.ROLE_SRC), np.flatnonzero(role == O.ROLE_DST)
    xn = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    for s_ in src:
        sims = xn[dst] @ xn[s_]
        best = dst[int(np.argmax(sims))]
        if m.match_dst[s_] != best:  # only a float near-tie may differ
            assert abs(sims.max() - float(xn[m.match_dst[s_]] @ xn[s_])) < 1e-6
        assert m.rep[s_] == m.rep[m.match_dst[s_]]
    alone = np.flatnonzero((role == O.ROLE_PROTECT) | (role == O.ROLE_SPECIAL))
    assert np.all(m.rep[alone] == alone)
    assert len(np.unique(m.rep)) == len(dst) + len(alone)
    for d in dst:  # a destination's group is itself and its sources; rep = smallest id
        mem = np.r_[d, src[m.match_dst[src] == d]]
        assert np.all(m.rep[mem] == mem.min())


def test_ga_protect_all_is_exact_attention():
    """100 % protected: nothing merges, so the layer is exact attention."""
    w = gen.WORKLOADS["tiny"].with_(frames=2, grid_h=6, grid_w=6, n_special=1, outlier_pct=10.0)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    p = O.Params(**{**p.__dict__, "partition": 1, "protect_pct": 100.0})
    tr = O.layer(x["q"], x["k"], x["v"], p)
    for h in range(w.heads):
        ref = O.attention(x["q"][h], x["k"][h], x["v"][h], p.scale)
        assert np.abs(tr.out[h] - ref).max() <= 1e-5


# --------------------------------------------------------------------------
# Cached-index layer (LiteVGGT page, key design 3: merge indices of one layer
# are reused by the next ones; only the means are recomputed)
# --------------------------------------------------------------------------
def test_layer_cached_with_the_layers_own_indices_equals_the_layer():
    """Reusing a layer's own final query partition and key partition on the
    same inputs reproduces that layer's output bit for bit; swapping the two
    partitions (a plausible slip) does not."""
    for part in (0, 1):
        p = _small(pct=15.0) if part == 0 else _ga_params(heads=2, outlier_pct=15.0)
        q, k, v = (_rand_qkv(p, 21) if part == 0 else
                   [np.random.default_rng(21 + i).standard_normal((2, p.n_tokens, 64)).astype(np.float32)
                    for i in range(3)])
        tr = O.layer(q, k, v, p)
        got = O.layer_cached(q, k, v, p, tr.q_final_rep, tr.k_rep)
        assert np.array_equal(got, tr.out)
        rows = np.array([0, 3, p.n_tokens - 1])
        # a row subset runs the fp64 products with other BLAS blocking: equal to rounding
        assert np.abs(O.layer_cached(q, k, v, p, tr.q_final_rep, tr.k_rep, rows=rows) - tr.out[:, rows]).max() < 1e-12
        assert np.array_equal(O.layer_cached(q, k, v, p, tr.q_final_rep, tr.k_rep, out_heads=[1]), tr.out[[1]])
        swapped = O.layer_cached(q, k, v, p, tr.k_rep, tr.q_final_rep)
        assert not np.allclose(swapped, tr.out)


def test_layer_cached_hand_example_scaled_inputs():
    """On the hand block, the cached layer with the hand-derived partitions
    (p = 25 %) and inputs scaled by 2 equals SDPA on twice the hand-derived
    merged rows (means are linear; the scale is exact in fp32)."""
    ex, p, q, k, v = _hand()
    e = ex["expected"]
    rep_of = lambda groups: np.array([min(g) for n in range(8) for g in groups if n in g])
    qf = rep_of(e["p25"]["final_groups"])
    kr = rep_of(e["groups"])  # k == q: the key groups are the query groups before outliers
    got = O.layer_cached(2 * q, 2 * k, 2 * v, p, [qf], [kr])[0]
    fq = e["p25"]["final_q"]
    slots = sorted(int(r) for r in fq)
    Q = 2 * np.array([[_expr(x) for x in fq[str(r)]] for r in slots])
    kreps = sorted(int(r) for r in e["v_means"])
    K = 2 * np.array([[_expr(x) for x in e["q_means"][str(r)]] for r in kreps])
    V = 2 * np.array([[_expr(x) for x in e["v_means"][str(r)]] for r in kreps])
    o = _sdpa64(Q, K, V, 1.0)
    want = np.stack([o[slots.index(int(qf[n]))] for n in range(8)])
    assert np.allclose(got, want, atol=1e-6)


def test_layer_cached_value_shift_and_singletons():
    """A constant added to every value row shifts every output row by that
    constant (softmax weights sum to one and a mean of shifted rows is the
    shifted mean); singleton partitions give exact attention (fp64 SDPA)."""
    p = _small(pct=10.0)
    q, k, v = _rand_qkv(p, 22)
    tr = O.layer(q, k, v, p)
    c = np.float32(0.5)  # exact in fp32 next to values of this size
    base = O.layer_cached(q, k, v, p, tr.q_final_rep, tr.k_rep)
    shifted = O.layer_cached(q, k, v + c, p, tr.q_final_rep, tr.k_rep)
    assert np.abs(shifted - base - c).max() < 1e-6
    ident = [np.arange(p.n_tokens)] * p.heads
    single = O.layer_cached(q, k, v, p, ident, ident)
    for h in range(p.heads):
        assert np.abs(single[h] - _sdpa64(q[h], k[h], v[h], p.scale)).max() < 1e-12


def test_layer_cached_head_permutation():
    """Heads are independent: permuting the heads of the inputs and of the
    cached partitions permutes the outputs."""
    p = _small(heads=3, pct=10.0)
    q, k, v = _rand_qkv(p, 23)
    tr = O.layer(q, k, v, p)
    perm = [2, 0, 1]
    got = O.layer_cached(q[perm], k[perm], v[perm], p, [tr.q_final_rep[h] for h in perm],
                         [tr.k_rep[h] for h in perm])
    assert np.array_equal(got, tr.out[perm])


# --------------------------------------------------------------------------
# Head-shared global matching (HTTM page, research background and key designs
# 1-2: one merge topology for every head, matched over the whole sequence
# with a 25 % destination / 75 % source split)
# --------------------------------------------------------------------------
def _gm_params(**kw):
    base = dict(heads=2, d_head=8, frames=3, grid_h=3, grid_w=4, n_special=1, n_s=4, n_t=2, q_ratio=0.5,
                kv_ratio=0.5, outlier_pct=10.0, partition=2)
    base.update(kw)
    return O.Params(**base)


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(31).standard_normal(20000).astype(np.float32) * 3
    x = np.r_[x, np.float32(1 + 2 ** -8), np.float32(1 + 3 * 2 ** -8), np.float32(-0.0), np.float32(0.0)]
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.round_bf16_rne(x).view(np.uint32), want.view(np.uint32))


def test_global_match_is_one_block_over_all_patches():
    """With one head the shared metric is that head's keys, and global
    matching equals the block-local matching of the same keys with a single
    block of every patch in original order (n_s = H*W, n_t = F,
    frame-major), stride 4 and the same ratio."""
    for ratio in (0.3, 0.5, 0.75):
        p2 = _gm_params(heads=1, frames=4, grid_h=5, grid_w=6, kv_ratio=ratio)
        p0 = O.Params(**{**p2.__dict__, "partition": 0, "n_s": 30, "n_t": 4, "q_dst_stride": 4, "kv_dst_stride": 4,
                         "q_ratio": ratio})
        assert len(O.blocks(p0)) == 1
        q, k, v = _rand_qkv(p2, 41)
        g = O.global_match(O.head_shared_metric(k, False), p2, ratio)
        b = O.match_stream(k[0], p0, ratio, 4)
        for f in ("rep", "match_dst", "selected", "is_src"):
            assert np.array_equal(getattr(g, f), getattr(b, f)), f
        assert np.array_equal(g.score[g.is_src], b.score[b.is_src])
        # with q = k the whole layer is the block-local layer
        t2 = O.layer(k, k, v, p2)
        t0 = O.layer(k, k, v, p0)
        assert np.array_equal(t2.out, t0.out)


def test_head_shared_metric_is_the_head_mean():
    """The metric is the mean key over heads: equal heads give that head back
    exactly (h = 2), and small integer keys give exact means; every head's
    query and key partitions are the one shared partition."""
    p = _gm_params(heads=2)
    q, k, v = _rand_qkv(p, 42)
    k2 = np.stack([k[0], k[0]])
    assert np.array_equal(O.head_shared_metric(k2, False), k[0])
    ki = np.random.default_rng(43).integers(-8, 8, size=(4, p.n_tokens, 8)).astype(np.float32)
    assert np.array_equal(O.head_shared_metric(ki, False), ki.astype(np.float64).mean(0).astype(np.float32))
    tr = O.layer(q, k, v, p)
    shared = O.global_match(O.head_shared_metric(k, False), p, p.kv_ratio)
    for h in range(p.heads):
        assert np.array_equal(tr.k_rep[h], shared.rep)
        assert np.array_equal(tr.q_match[h].rep, shared.rep)
    # the outlier restore still acts per head on the shared query groups
    assert tr.outlier.sum() == O.outlier_budget(p)


@pytest.mark.parametrize("seed", range(4))
def test_global_match_brute_force(seed):
    """Double-loop cosine similarity, per-source argmax and exhaustive top-r
    over all source subsets on a tiny sequence (12 patches)."""
    rng = np.random.default_rng(200 + seed)
    p = O.Params(heads=3, d_head=3, frames=3, grid_h=1, grid_w=4, n_special=1, n_s=4, n_t=3, q_ratio=0.5,
                 kv_ratio=[0.25, 0.5, 0.6, 0.75][seed], outlier_pct=0.0, partition=2)
    k = rng.integers(-4, 5, size=(3, p.n_tokens, 3)).astype(np.float32)
    m = O.head_shared_metric(k, False)
    patches = np.flatnonzero(~O.is_special(p))
    g = O.global_match(m, p, p.kv_ratio)
    match, score, sel = _brute_block(m[patches], 4, p.kv_ratio)
    for i, j in match.items():
        assert g.match_dst[patches[i]] == patches[j]
        assert abs(g.score[patches[i]] - score[i]) < 1e-6
    assert {i for i in range(len(patches)) if g.selected[patches[i]]} == sel


# ---------------------------------------------------------------- FP8 scores (R41-R44)
def _torch_e4m3(x):
    """Library reference: torch's float8_e4m3fn conversion (nearest, ties to even)."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _finite_e4m3():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return codes[np.isfinite(codes)]


def test_e4m3_round_matches_torch():
    """Against torch's e4m3 conversion: a log-uniform sweep over the normal
    and subnormal range, every finite code (unchanged) and every midpoint
    between neighbouring codes (to the even mantissa)."""
    rng = np.random.default_rng(41)
    x = (rng.standard_normal(400_000) * np.exp2(rng.uniform(-14, 8, 400_000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    assert np.array_equal(O.e4m3_round(x), _torch_e4m3(x))
    fin = _finite_e4m3()
    assert len(fin) == 254 and np.array_equal(O.e4m3_round(fin), fin)
    pos = np.unique(np.abs(fin))
    mids = np.concatenate([(pos[:-1] + pos[1:]) / 2, -(pos[:-1] + pos[1:]) / 2])
    assert np.array_equal(O.e4m3_round(mids), _torch_e4m3(mids))
    with pytest.raises(ValueError):
        O.e4m3_round(np.array([449.0]))


def test_e4m3_round_hand_values():
    """Hand-derived: spacing 2^-3 in [1, 2), ties to the even mantissa, the
    subnormal spacing 2^-9 below 2^-6, and the top binade [256, 448]."""
    cases = [(1.0625, 1.0), (1.1875, 1.25), (1.0625 + 2.0 ** -20, 1.125), (2.0 ** -10, 0.0),
             (3 * 2.0 ** -10, 2.0 ** -8), (2.0 ** -6 + 2.0 ** -10, 2.0 ** -6), (-0.3, -0.3125),
             (248.0, 256.0), (240.0, 240.0), (440.0, 448.0), (0.0, 0.0)]
    x = np.array([c[0] for c in cases])
    assert O.e4m3_round(x).tolist() == [c[1] for c in cases]


def test_fp8_exponent_lands_amax_in_128_256():
    rng = np.random.default_rng(42)
    amax = np.concatenate([np.exp2(rng.uniform(-120, 120, 5000)), np.exp2(np.arange(-120, 121.0))])
    e = O.fp8_exponent(amax)
    s = np.ldexp(amax, e)
    assert ((s >= 128) & (s < 256)).all()
    assert O.fp8_exponent(np.array([0.0, 1.0, 255.9, 256.0])).tolist() == [0, 7, 0, -1]
    assert O.fp8_exponent(np.array([2.0 ** -130, 2.0 ** 140])).tolist() == [127, -127]  # clamped


def _brute_fp8_attention(q, k2, v):
    """Loops: exponents found by search, elements rounded by torch, exact
    products (e4m3 products and their sums are exact in fp64 here), base-2
    softmax."""
    def expo(amax):
        if amax == 0:
            return 0
        for e in range(-127, 128):
            if 128 <= amax * 2.0 ** e < 256:
                return e
        raise AssertionError
    ek = expo(float(np.abs(k2).max()))
    k8 = _torch_e4m3(np.asarray(k2, np.float64) * 2.0 ** ek)
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        eq = expo(float(np.abs(q[i]).max()))
        q8 = _torch_e4m3(np.asarray(q[i], np.float64) * 2.0 ** eq)
        s = [sum(float(q8[d]) * float(k8[j, d]) for d in range(q.shape[1])) * 2.0 ** -(eq + ek)
             for j in range(k2.shape[0])]
        m = max(s)
        p = [2.0 ** (x - m) for x in s]
        out[i] = sum(pj * np.asarray(v[j], np.float64) for j, pj in enumerate(p)) / sum(p)
    return out


@pytest.mark.parametrize("seed", range(3))
def test_attention_fp8_brute_force(seed):
    rng = np.random.default_rng(43 + seed)
    q = (rng.standard_normal((6, 16)) * np.exp2(rng.uniform(-3, 3, (6, 1)))).astype(np.float32)
    k2 = (0.4 * rng.standard_normal((9, 16))).astype(np.float32)
    v = rng.standard_normal((9, 8)).astype(np.float32)
    got = O.attention_fp8(q, k2, v)
    assert np.abs(got - _brute_fp8_attention(q, k2, v)).max() < 1e-12
    # quantisation is really there: the exact base-2 softmax differs
    exact = _sdpa64(q, k2.astype(np.float64) * math.log(2.0), v, 1.0)
    assert np.abs(got - exact).max() > 1e-6


def test_attention_fp8_exact_on_representable_operands():
    """Integers of at most 4 significant bits stay e4m3 values after any
    power-of-two scale: the FP8 scores are then the exact scores, and the
    output is the fp64 attention (torch sdpa with scale ln 2 for base 2)."""
    rng = np.random.default_rng(44)
    q = rng.integers(-15, 16, (7, 16)).astype(np.float32) * np.exp2(rng.integers(-4, 4, (7, 1))).astype(np.float32)
    k2 = rng.integers(-15, 16, (11, 16)).astype(np.float32) / 64
    v = rng.standard_normal((11, 8)).astype(np.float32)
    assert np.abs(O.attention_fp8(q, k2, v) - _sdpa64(q, k2.astype(np.float64) * math.log(2.0), v, 1.0)).max() < 1e-12


def test_attention_fp8_power_of_two_invariance():
    """Queries times 2^a and keys times 2^-a: every exponent absorbs the
    factor, no code changes, the output is bit-identical.  A factor that is
    not a power of two changes codes and the output."""
    rng = np.random.default_rng(45)
    q = rng.standard_normal((20, 64)).astype(np.float32)
    k2 = (0.2 * rng.standard_normal((50, 64))).astype(np.float32)
    v = rng.standard_normal((50, 64)).astype(np.float32)
    base = O.attention_fp8(q, k2, v)
    for a in (-3, 5):
        assert np.array_equal(O.attention_fp8(q * np.float32(2.0 ** a), k2 * np.float32(2.0 ** -a), v), base)
    assert not np.array_equal(O.attention_fp8(q * np.float32(1.1), k2 / np.float32(1.1), v), base)


def test_fp8_scores_error_bound():
    """|S8 - S| <= sum_d (|dq_d| |k^_d| + |q_d| |dk_d|), where each element's
    rounding error is at most 2^-4 of its scaled magnitude plus 2^-10 (half
    the subnormal spacing), descaled."""
    rng = np.random.default_rng(46)
    q = (rng.standard_normal((40, 64)) * np.exp2(rng.uniform(-4, 4, (40, 1)))).astype(np.float64)
    k2 = (0.3 * rng.standard_normal((70, 64))).astype(np.float64)
    s8 = O.fp8_scores(q, k2)
    s = q @ k2.T
    eq = np.array([math.frexp(a)[1] for a in np.abs(q).max(axis=1)])  # amax in [2^(e-1), 2^e)
    ek = math.frexp(float(np.abs(k2).max()))[1]
    dq = 2.0 ** -4 * np.abs(q) + 2.0 ** -10 * 2.0 ** (eq[:, None] - 8)
    dk = 2.0 ** -4 * np.abs(k2) + 2.0 ** -10 * 2.0 ** (ek - 8)
    bound = dq @ (np.abs(k2) + dk).T + np.abs(q) @ dk.T
    assert (np.abs(s8 - s) <= bound).all()
    assert np.abs(s8 - s).max() > 0


def test_layer_fp8_no_merge_is_brute_force_fp8_attention():
    """Merge ratios 0: every slot is one token, so the FP8 layer's head
    output is the brute-force FP8 attention of the stored bf16 operands --
    queries rounded to bf16, keys times fp32(scale) * fp32(log2 e) rounded
    to bf16 (R44)."""
    p = _small(heads=1, frames=2, gh=3, gw=3, sp=1, n_s=4, n_t=2, qr=0.0, kr=0.0, pct=0.0,
               softmax_scale=0.3, attn_fp8=True)
    p8 = p
    q, k, v = _rand_qkv(p, 47)
    tr = O.layer(q, k, v, p8)
    ks = np.float32(np.float32(0.3) * np.float32(1.4426950408889634))
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    ref = _brute_fp8_attention(bf(q[0]), bf((k[0] * ks).astype(np.float32)), bf(v[0]))
    assert np.abs(tr.out[0] - ref).max() < 1e-12
    # the bf16 layer on the same inputs differs (the scores are quantised)
    p16 = O.Params(**{**p.__dict__, "attn_fp8": False})
    assert np.abs(O.layer(q, k, v, p16).out[0] - tr.out[0]).max() > 1e-5


def test_layer_fp8_close_to_bf16_layer():
    """The FP8 layer's partitions are the bf16 layer's (FP8 enters only the
    attention scores), and its output stays near it on redundant tokens."""
    p = _small(pct=10.0, softmax_scale=0.0)
    q, k, v = _rand_qkv(p, 48)
    a = O.layer(q, k, v, p)
    b = O.layer(q, k, v, O.Params(**{**p.__dict__, "attn_fp8": True}))
    for h in range(p.heads):
        assert np.array_equal(a.q_final_rep[h], b.q_final_rep[h]) and np.array_equal(a.k_rep[h], b.k_rep[h])
    rel = np.sqrt(((a.out - b.out) ** 2).mean()) / np.sqrt((a.out ** 2).mean())
    assert 0 < rel < 0.1
