"""Plain CPU oracle of HTTM's head-wise temporal token-merged global attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this module.  It shares no
code with the HIP path (``token_merged_global_amd``) and never serves as a
fallback for it.

It is written from "HTTM: Head-wise Temporal Token Merging for Faster VGGT"
(papernotes.org summary, sections "key design 1-3", "overall framework",
"training strategy / settings") and the merge formula and index-cache
description of "LiteVGGT: Boosting Vanilla VGGT via Geometry-aware Cached Token
Merging" (papernotes.org summary, "key design 3").  Each function cites the
passage it follows.  Where the pages leave a step open the reading taken is
stated next to the code and collected in the design notes as R1..R30.

Precision.  Steps whose floating-point result decides an integer (the cosine
argmax, the top-r order, the deviation that picks outliers) run in fp32, the
precision the kernels take those decisions in.  Means are fp32 sums taken in
ascending original token index followed by one fp32 division; deviations are
fp32 sums of squares taken in ascending channel order followed by a correctly
rounded square root.  Attention runs in fp64 (it decides nothing).

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
(hand example with closed forms, exact attention limits against
``torch.nn.functional.scaled_dot_product_attention``, brute force on tiny
blocks, invariants).  Absolute layer outputs at the VGGT-shaped sizes are
pinned only through those properties ("parity unpinned" for the absolute
values; see the test module's header).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

EPS_NORM = 1e-12  # R10: F.normalize convention for zero rows


# --------------------------------------------------------------------------
# Parameters and the token map
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Params:
    """Layer parameters (HTTM page, "training strategy / settings")."""

    heads: int
    d_head: int
    frames: int
    grid_h: int
    grid_w: int
    n_special: int
    n_s: int
    n_t: int
    q_ratio: float
    kv_ratio: float
    outlier_pct: float
    q_dst_stride: int = 0
    kv_dst_stride: int = 0
    block_order: int = 0  # 0 frame-major (R3), 1 frame-minor
    softmax_scale: float = 0.0  # 0 -> 1/sqrt(d_head) (R21)
    partition: int = 0  # 0 HTTM temporal blocks; 1 geometry-aware three-class partition (R31);
    #                     2 one head-shared topology from global matching (R37-R40)
    protect_pct: float = 10.0  # geometry-aware partition: percent of each frame's patches protected
    attn_fp8: bool = False  # attention scores from FP8 (OCP e4m3) queries and keys (R41-R44)

    @property
    def tokens_per_frame(self) -> int:
        return self.n_special + self.grid_h * self.grid_w

    @property
    def n_tokens(self) -> int:
        return self.frames * self.tokens_per_frame

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.d_head)

    @staticmethod
    def from_workload(w) -> "Params":
        return Params(heads=w.heads, d_head=w.d_head, frames=w.frames, grid_h=w.grid_h,
                      grid_w=w.grid_w, n_special=w.n_special, n_s=w.n_s, n_t=w.n_t,
                      q_ratio=w.q_ratio, kv_ratio=w.kv_ratio, outlier_pct=w.outlier_pct,
                      q_dst_stride=w.q_dst_stride, kv_dst_stride=w.kv_dst_stride,
                      block_order=getattr(w, "block_order", 0), softmax_scale=w.softmax_scale,
                      partition=getattr(w, "partition", 0), protect_pct=getattr(w, "protect_pct", 10.0),
                      attn_fp8=bool(getattr(w, "attn_fp8", False)))


def dst_stride(ratio: float, given: int = 0) -> int:
    """Destination stride s (R8).

    The configs ask for "dst every 4th" and also a 90 % query merge, which one
    bipartite round cannot give with a quarter of the tokens as destinations.
    Reading: s = max(4, ceil(1/(1-ratio) - 1e-9)), so every fourth token stays
    a destination wherever that is feasible and the 90 % setting gives the
    page's 20 % final query length (HTTM page, settings).
    """
    if given > 0:
        return int(given)
    return max(4, int(math.ceil(1.0 / (1.0 - ratio) - 1e-9)))


def is_special(p: Params) -> np.ndarray:
    """Token n = f*T + t is special iff t < n_special (R6)."""
    t = np.arange(p.n_tokens) % p.tokens_per_frame
    return t < p.n_special


# --------------------------------------------------------------------------
# Step 1: temporal reordering into spatio-temporal blocks
# --------------------------------------------------------------------------
@dataclass
class Block:
    g: int  # temporal group
    a: int  # spatial run
    f0: int
    nf: int
    j0: int
    run: int
    tokens: np.ndarray  # original token ids in block order

    @property
    def n(self) -> int:
        return len(self.tokens)


def blocks(p: Params) -> List[Block]:
    """Spatio-temporal merge blocks (HTTM page, key design 2).

    Tokens of the same spatial region (a run of n_s raster-order patches, R4)
    in n_t adjacent frames (R5: the last group may be shorter) are stacked into
    one block of n_b = n_s * n_t tokens.  Inside a block the stack is
    frame-major (R3); blocks are ordered by temporal group, then spatial run.
    Special tokens are not reordered (R6).
    """
    HW = p.grid_h * p.grid_w
    T = p.tokens_per_frame
    A = -(-HW // p.n_s)
    G = -(-p.frames // p.n_t)
    out = []
    for g in range(G):
        f0 = g * p.n_t
        nf = min(p.n_t, p.frames - f0)
        for a in range(A):
            j0 = a * p.n_s
            run = min(p.n_s, HW - j0)
            f = np.arange(f0, f0 + nf)
            j = np.arange(j0, j0 + run)
            if p.block_order == 0:
                tok = (f[:, None] * T + p.n_special + j[None, :]).reshape(-1)
            else:
                tok = (f[None, :] * T + p.n_special + j[:, None]).reshape(-1)
            out.append(Block(g, a, f0, nf, j0, run, tok.astype(np.int64)))
    return out


def reorder_permutation(p: Params) -> np.ndarray:
    """pi: reordered position -> original token id, over the patch tokens."""
    return np.concatenate([b.tokens for b in blocks(p)])


# --------------------------------------------------------------------------
# Steps 2-3: per-head block matching and top-r selection
# --------------------------------------------------------------------------
def row_normalize(x: np.ndarray) -> np.ndarray:
    """RowNorm (HTTM page, key design 1), fp32, zero rows map to zero (R10)."""
    x = x.astype(np.float32)
    nrm = np.sqrt(np.sum(x * x, axis=1, dtype=np.float32)).astype(np.float32)
    return (x / np.maximum(nrm, np.float32(EPS_NORM))[:, None]).astype(np.float32)


def block_similarity(xb: np.ndarray, s: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Sim = RowNorm(S) . RowNorm(D)^T of one block (HTTM page, key design 1).

    Block positions i with i mod s == 0 are destinations D, the rest sources S
    (R7, R8).  Returns (dst positions, src positions, fp32 sim [|S|][|D|]).
    """
    n = xb.shape[0]
    pos = np.arange(n)
    dpos = pos[pos % s == 0]
    spos = pos[pos % s != 0]
    sim = (row_normalize(xb[spos]) @ row_normalize(xb[dpos]).T).astype(np.float32)
    return dpos, spos, sim


def match_block(xb: np.ndarray, s: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Bipartite cosine matching inside one block (HTTM page, key design 1).

    Every source keeps only its most similar destination, ties to the smaller
    destination position (R11).  Returns (dst positions, src positions,
    matched dst position per src, score per src).
    """
    dpos, spos, sim = block_similarity(xb, s)
    if len(spos) == 0:
        return dpos, spos, np.zeros(0, np.int64), np.zeros(0, np.float32)
    j = np.argmax(sim, axis=1)  # first maximum = smallest dst position
    score = sim[np.arange(len(spos)), j] + np.float32(0.0)  # canonical +0
    return dpos, spos, dpos[j], score.astype(np.float32)


def merge_count(ratio: float, n: int, n_src: int) -> int:
    """r = min(|S|, floor(ratio * n + 1e-9)) in binary64 (R2, R9)."""
    return min(n_src, int(math.floor(ratio * n + 1e-9)))


def select_top_r(score: np.ndarray, spos: np.ndarray, r: int) -> np.ndarray:
    """Boolean mask of the r sources with the highest score (HTTM page, key design 1).

    Ties go to the smaller source position (R11).
    """
    order = np.lexsort((spos, -score.astype(np.float64)))
    sel = np.zeros(len(spos), dtype=bool)
    sel[order[:r]] = True
    return sel


@dataclass
class StreamMatch:
    """Per-head matching result of one stream (q or k) over all blocks."""

    rep: np.ndarray  # [N] canonical group id = smallest original id in the group
    match_dst: np.ndarray  # [N] original id of the matched dst for sources, -1 otherwise
    score: np.ndarray  # [N] score for sources, nan otherwise
    selected: np.ndarray  # [N] bool, source chosen among the top-r
    is_src: np.ndarray  # [N] bool


def match_stream(x: np.ndarray, p: Params, ratio: float, stride: int) -> StreamMatch:
    """Steps 2-4 for one head and one stream: match, select, group.

    Groups are {d} u {selected s : m(s) = d} for each destination d, plus one
    singleton per unselected source and per special token (HTTM page, key
    design 1; R6, R12).
    """
    N = p.n_tokens
    s = dst_stride(ratio, stride)
    rep = np.arange(N, dtype=np.int64)
    mdst = np.full(N, -1, dtype=np.int64)
    score = np.full(N, np.nan, dtype=np.float32)
    selected = np.zeros(N, dtype=bool)
    is_src = np.zeros(N, dtype=bool)
    for b in blocks(p):
        tok = b.tokens
        dpos, spos, mpos, sc = match_block(x[tok], s)
        r = merge_count(ratio, b.n, len(spos))
        sel = select_top_r(sc, spos, r)
        src_tok = tok[spos]
        dst_of_src = tok[mpos]
        is_src[src_tok] = True
        mdst[src_tok] = dst_of_src
        score[src_tok] = sc
        selected[src_tok] = sel
        # group id: the smallest original id among the dst and its selected sources
        g = tok.copy()  # default: own id
        g[spos[sel]] = dst_of_src[sel]  # temporarily label by dst id
        lab = g  # label per block position: dst id for dst and selected src
        # canonical representative = min original id over members of each label
        labs, inv = np.unique(lab, return_inverse=True)
        mins = np.full(len(labs), np.iinfo(np.int64).max, dtype=np.int64)
        np.minimum.at(mins, inv, tok)
        rep[tok] = mins[inv]
    return StreamMatch(rep=rep, match_dst=mdst, score=score, selected=selected, is_src=is_src)


# --------------------------------------------------------------------------
# Geometry-aware three-class partition (an alternative to steps 2-4)
# --------------------------------------------------------------------------
# "LiteVGGT: Boosting Vanilla VGGT via Geometry-aware Cached Token Merging",
# key designs 1-3: a geometry score per token, three token classes (protected
# high-score tokens, destinations, sources) and a cosine match of every
# source to its most similar destination.  Used here, like HTTM's matching,
# per head and per stream (R1).  Readings R31-R36 (design notes).


def _box3_sum(a: np.ndarray, axis: int) -> np.ndarray:
    """Sum of each element and its existing neighbours along `axis` (fp32):
    (left + centre) + right, in ascending order, clipped at the ends."""
    a = np.moveaxis(a, axis, 0)
    t = a.copy()
    if a.shape[0] > 1:
        t[1:] = (a[:-1] + a[1:]).astype(np.float32)  # left + centre
        t[:-1] = (t[:-1] + a[1:]).astype(np.float32)  # ... + right
    return np.moveaxis(t, 0, axis)


def token_variance_map(x: np.ndarray, p: Params) -> np.ndarray:
    """Token variance map v (LiteVGGT page, key design 1; variance half, R31).

    Patch tokens of each frame are laid on their grid; v of a token is the
    mean over channels of the variance of the features in its 3x3
    neighbourhood (average pooling of x and x^2, windows clipped at the grid
    edge, R32).  fp32 in a fixed order (R33): per channel, each row's
    available cells are summed left to right, then the available rows top to
    bottom (for x and for x*x); var = s2/cnt - (s1/cnt)^2; v = (sum of var
    over channels in ascending order) / d.  Special tokens get 0 (they are
    never merged).
    """
    H_, W_ = p.grid_h, p.grid_w
    T = p.tokens_per_frame
    d = x.shape[1]
    ncol = np.full(W_, 3.0 if W_ > 2 else float(min(W_, 2)), np.float32)
    ncol[[0, -1]] = float(min(W_, 2))
    nrow = np.full(H_, 3.0 if H_ > 2 else float(min(H_, 2)), np.float32)
    nrow[[0, -1]] = float(min(H_, 2))
    cnt = (nrow[:, None] * ncol[None, :])[:, :, None].astype(np.float32)
    v = np.zeros(p.n_tokens, dtype=np.float32)
    for f in range(p.frames):
        g = x[f * T + p.n_special:(f + 1) * T].astype(np.float32).reshape(H_, W_, d)
        s1 = _box3_sum(_box3_sum(g, 1), 0)
        s2 = _box3_sum(_box3_sum((g * g).astype(np.float32), 1), 0)
        m = (s1 / cnt).astype(np.float32)
        var = ((s2 / cnt).astype(np.float32) - (m * m).astype(np.float32)).astype(np.float32)
        acc = np.zeros((H_, W_), dtype=np.float32)
        for ch in range(d):
            acc = (acc + var[:, :, ch]).astype(np.float32)
        v[f * T + p.n_special:(f + 1) * T] = (acc / np.float32(d)).astype(np.float32).reshape(-1)
    return v


ROLE_SRC, ROLE_DST, ROLE_PROTECT, ROLE_SPECIAL = 0, 1, 2, 3


def ga_roles(v: np.ndarray, p: Params) -> np.ndarray:
    """Three token classes (LiteVGGT page, key design 2; R34, R35).

    Per frame the k = floor(protect_pct/100 * H*W + 1e-9) patches with the
    highest score are protected (ties to the smaller patch index).  Every
    unprotected patch of the first frame is a destination; in every other
    frame, each 2x2 cell of the grid (clipped at odd edges) contributes its
    unprotected patch with the lowest score (ties to the smaller patch index),
    if it has one.  The remaining patches are sources; specials keep their own
    role.
    """
    H_, W_ = p.grid_h, p.grid_w
    T, HW = p.tokens_per_frame, p.grid_h * p.grid_w
    k = int(math.floor(p.protect_pct / 100.0 * HW + 1e-9))
    role = np.full(p.n_tokens, ROLE_SRC, dtype=np.int8)
    for f in range(p.frames):
        base = f * T
        role[base:base + p.n_special] = ROLE_SPECIAL
        vf = v[base + p.n_special:base + T]
        j = np.arange(HW)
        order = np.lexsort((j, -vf.astype(np.float64)))  # score desc, index asc
        prot = np.zeros(HW, dtype=bool)
        prot[order[:k]] = True
        rf = np.full(HW, ROLE_SRC, dtype=np.int8)
        rf[prot] = ROLE_PROTECT
        if f == 0:
            rf[~prot] = ROLE_DST
        else:
            for cy in range(0, H_, 2):
                for cx in range(0, W_, 2):
                    cell = [y * W_ + x for y in range(cy, min(cy + 2, H_)) for x in range(cx, min(cx + 2, W_))]
                    cand = [c for c in cell if not prot[c]]
                    if cand:
                        best = min(cand, key=lambda c: (float(vf[c]), c))
                        rf[best] = ROLE_DST
        role[base + p.n_special:base + T] = rf
    return role


def ga_similarity(x: np.ndarray, src: np.ndarray, dst: np.ndarray) -> np.ndarray:
    """Cosine of every listed source with every listed destination
    (LiteVGGT page, key design 3): products of RowNorm rows, fp32."""
    return (row_normalize(x[src]) @ row_normalize(x[dst]).T).astype(np.float32)


def ga_match_stream(x: np.ndarray, p: Params, chunk: int = 4096) -> StreamMatch:
    """Geometry-aware grouping of one head and stream (LiteVGGT page, key designs 2-3).

    Every source joins its most similar destination over the whole sequence
    (cosine of RowNorm rows, fp32; ties to the smaller destination id, R36);
    groups are each destination with its sources, and singletons for
    protected and special tokens.
    """
    N = p.n_tokens
    role = ga_roles(token_variance_map(x, p), p)
    src = np.flatnonzero(role == ROLE_SRC)
    dst = np.flatnonzero(role == ROLE_DST)
    rep = np.arange(N, dtype=np.int64)
    mdst = np.full(N, -1, dtype=np.int64)
    score = np.full(N, np.nan, dtype=np.float32)
    if len(src) and len(dst):
        for c0 in range(0, len(src), chunk):
            sc = src[c0:c0 + chunk]
            sim = ga_similarity(x, sc, dst)
            jj = np.argmax(sim, axis=1)  # first maximum = smallest destination id
            mdst[sc] = dst[jj]
            score[sc] = sim[np.arange(len(sc)), jj] + np.float32(0.0)
        m = mdst[src]
        # group of a source: its destination's; rep = min id over the group
        grp = rep.copy()
        grp[src] = m
        mins = np.arange(N, dtype=np.int64)
        np.minimum.at(mins, grp, np.arange(N, dtype=np.int64))
        rep = mins[grp]
    is_src = role == ROLE_SRC
    return StreamMatch(rep=rep, match_dst=mdst, score=score, selected=is_src.copy(), is_src=is_src)


# --------------------------------------------------------------------------
# Head-shared global matching (the merging the HTTM page contrasts itself with)
# --------------------------------------------------------------------------
# HTTM page, research background and key design 1: ToMe-style merging (as
# FastVGGT uses it) applies one merge topology to every head and matches over
# the whole long sequence; key design 2 prices that global matching at about
# 0.19 N^2 d_head FLOPs for a 25 % destination / 75 % source split.
# Readings R37-R40 (design notes).
GM_STRIDE = 4  # R38: every 4th patch token is a destination (25 % / 75 %)


def round_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Nearest bf16 value of each fp32 value (ties to even), as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def head_shared_metric(k: np.ndarray, bf16: bool) -> np.ndarray:
    """The token feature one shared topology is matched on (R37): the key
    vectors averaged over heads -- an fp32 sum in ascending head order and
    one fp32 division by h -- rounded to bf16 (nearest, ties to even) in a
    bf16 layer, whose similarity takes bf16 operands."""
    acc = np.zeros(k.shape[1:], dtype=np.float32)
    for i in range(k.shape[0]):
        acc = (acc + k[i]).astype(np.float32)
    m = (acc / np.float32(k.shape[0])).astype(np.float32)
    return round_bf16_rne(m) if bf16 else m


def global_match(x: np.ndarray, p: Params, ratio: float, chunk: int = 4096) -> StreamMatch:
    """Bipartite matching over the whole sequence (R38, R39).

    The patch tokens in their original order (frames, then raster patches;
    no temporal reordering) form one block; positions i = 0, 4, 8, ... are
    destinations, the rest sources.  Every source keeps its most similar
    destination (cosine of RowNorm rows, fp32; ties to the smaller position),
    the r = min(|S|, floor(ratio * P + 1e-9)) sources with the highest score
    merge (ties to the smaller position), and groups are each destination
    with its merged sources; other sources and specials stay alone.
    """
    N = p.n_tokens
    tok = np.flatnonzero(~is_special(p))
    pos = np.arange(len(tok))
    dpos, spos = pos[pos % GM_STRIDE == 0], pos[pos % GM_STRIDE != 0]
    rep = np.arange(N, dtype=np.int64)
    mdst = np.full(N, -1, dtype=np.int64)
    score = np.full(N, np.nan, dtype=np.float32)
    selected = np.zeros(N, dtype=bool)
    is_src = np.zeros(N, dtype=bool)
    if len(spos) and len(dpos):
        dn = row_normalize(x[tok[dpos]])
        m = np.empty(len(spos), dtype=np.int64)
        sc = np.empty(len(spos), dtype=np.float32)
        for c0 in range(0, len(spos), chunk):
            sim = (row_normalize(x[tok[spos[c0:c0 + chunk]]]) @ dn.T).astype(np.float32)
            j = np.argmax(sim, axis=1)  # first maximum = smallest destination position
            m[c0:c0 + chunk] = dpos[j]
            sc[c0:c0 + chunk] = sim[np.arange(len(j)), j] + np.float32(0.0)
        r = merge_count(ratio, len(tok), len(spos))
        sel = select_top_r(sc, spos, r)
        src_tok, dst_of_src = tok[spos], tok[m]
        is_src[src_tok] = True
        mdst[src_tok] = dst_of_src
        score[src_tok] = sc
        selected[src_tok] = sel
        lab = np.arange(N, dtype=np.int64)
        lab[src_tok[sel]] = dst_of_src[sel]
        mins = np.arange(N, dtype=np.int64)
        np.minimum.at(mins, lab, np.arange(N, dtype=np.int64))
        rep = mins[lab]
    return StreamMatch(rep=rep, match_dst=mdst, score=score, selected=selected, is_src=is_src)


# --------------------------------------------------------------------------
# Partitions and means
# --------------------------------------------------------------------------
@dataclass
class Partition:
    """Groups of one head: reps (sorted), start offsets, members (ascending ids)."""

    reps: np.ndarray
    starts: np.ndarray  # len(reps) + 1
    members: np.ndarray  # original ids, grouped by rep, ascending inside a group
    group_of: np.ndarray  # [N] index into reps

    @property
    def sizes(self) -> np.ndarray:
        return np.diff(self.starts)


def partition(rep: np.ndarray) -> Partition:
    n = np.arange(len(rep))
    order = np.lexsort((n, rep))
    r_sorted = rep[order]
    brk = np.flatnonzero(np.r_[True, r_sorted[1:] != r_sorted[:-1]])
    starts = np.r_[brk, len(rep)]
    reps = r_sorted[brk]
    gid_sorted = np.repeat(np.arange(len(reps)), np.diff(starts))
    group_of = np.empty(len(rep), dtype=np.int64)
    group_of[order] = gid_sorted
    return Partition(reps=reps, starts=starts, members=order.astype(np.int64), group_of=group_of)


def group_means(x: np.ndarray, part: Partition) -> np.ndarray:
    """Mean of each group's members (HTTM page, key design 1; LiteVGGT page, key design 3).

    x_d_up = (x_d + sum_{s in S_d} x_s) / (1 + |S_d|): fp32 sum in ascending
    original id (R13), then one fp32 division by the member count.
    """
    G = len(part.reps)
    sizes = part.sizes
    acc = np.zeros((G, x.shape[1]), dtype=np.float32)
    for rank in range(int(sizes.max()) if G else 0):
        gs = np.flatnonzero(sizes > rank)
        acc[gs] = (acc[gs] + x[part.members[part.starts[gs] + rank]]).astype(np.float32)
    return (acc / sizes.astype(np.float32)[:, None]).astype(np.float32)


def deviation(q: np.ndarray, part: Partition, means: np.ndarray) -> np.ndarray:
    """L2 distance of every query to the mean of its group (HTTM page, key design 3).

    Every member of a group has a deviation, its destination included (R14);
    unmerged tokens come out exactly 0.  fp32: differences, squares and a
    running sum over channels in ascending order, then a correctly rounded sqrt.
    """
    diff = (q - means[part.group_of]).astype(np.float32)
    sq = (diff * diff).astype(np.float32)
    acc = np.zeros(q.shape[0], dtype=np.float32)
    for c in range(q.shape[1]):
        acc = (acc + sq[:, c]).astype(np.float32)
    return np.sqrt(acc).astype(np.float32)


# --------------------------------------------------------------------------
# Step 5: cross-head adaptive outlier filter
# --------------------------------------------------------------------------
def outlier_budget(p: Params) -> int:
    """k_o = floor(p * h * N / 100 + 1e-9), N counting special tokens (R15, R16)."""
    return int(math.floor(p.outlier_pct * p.heads * p.n_tokens / 100.0 + 1e-9))


def select_outliers(delta: np.ndarray, k_o: int) -> np.ndarray:
    """Global top-k_o deviations over all heads and tokens (HTTM page, key design 3).

    Returns the mask M_o [h][N].  Ties go to the smaller flat index h*N + n (R17).
    """
    h, N = delta.shape
    flat = delta.reshape(-1).astype(np.float32)
    order = np.lexsort((np.arange(h * N), -flat.astype(np.float64)))
    m = np.zeros(h * N, dtype=bool)
    m[order[:k_o]] = True
    return m.reshape(h, N)


def restore_partition(q_rep: np.ndarray, outlier: np.ndarray) -> np.ndarray:
    """Final query partition after the outlier filter (HTTM page, key design 3).

    Each outlier leaves its group and becomes an independent token; a group
    keeps its remaining members; a group left empty disappears.  The group id
    stays the smallest remaining original id.
    """
    N = len(q_rep)
    n = np.arange(N)
    key = np.where(outlier, N + n, q_rep)  # outliers: own label, disjoint from group labels
    # recanonicalise the remaining groups to their smallest remaining member
    labs, inv = np.unique(key, return_inverse=True)
    mins = np.full(len(labs), np.iinfo(np.int64).max, dtype=np.int64)
    np.minimum.at(mins, inv, n)
    return mins[inv]


# --------------------------------------------------------------------------
# Step 6: attention on the shortened sequences, step 7: unmerge
# --------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              chunk: int = 2048) -> np.ndarray:
    """O = softmax(scale * Q K^T) V in fp64 with max subtraction (R20, R21)."""
    q64 = q.astype(np.float64)
    k64 = k.astype(np.float64)
    v64 = v.astype(np.float64)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for i in range(0, q.shape[0], chunk):
        s = (q64[i:i + chunk] @ k64.T) * scale
        s -= s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[i:i + chunk] = (e @ v64) / e.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# FP8 attention scores (LiteVGGT page, training strategy and ablations: FP8
# quantisation for inference; here an OCP e4m3 variant of our own)
# --------------------------------------------------------------------------
# Readings R41-R44 (design notes).  R41: e4m3 with 448 as the largest finite
# magnitude, round to nearest with ties to even.  R42: the merged queries and
# keys (the score product) are FP8; probabilities and merged values stay
# bf16; sums are exact here (fp32 on the device).  R43: power-of-two scales,
# one per query row and one per head's key matrix, each chosen so that the
# block's largest magnitude lands in [128, 256).  R44: what is quantised is
# the stored bf16 operand: the query mean, and the key mean times the softmax
# scale and log2(e) (scores in log2 units, softmax in base 2).
LOG2E = 1.4426950408889634
E4M3_MAX = 448.0


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Nearest OCP e4m3 value of every element, ties to even (R41), as fp64.

    A normal value in [2^e, 2^(e+1)) (e >= -6) has 3 fraction bits, so its
    grid spacing is 2^(e-3); below 2^-6 the subnormal spacing is 2^-9.
    Dividing by the spacing is exact, and numpy's round() takes exact halves
    to the even integer, which is the even mantissa.  Magnitudes above 448
    have no finite encoding; the scales of R43 never produce them.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if (a > E4M3_MAX).any():
        raise ValueError("value beyond the e4m3 range")
    _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1): the binade is 2^(ex-1)
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, e - 3)
    return np.copysign(np.round(a / q) * q, x)


def fp8_exponent(amax: np.ndarray) -> np.ndarray:
    """Scale exponent e of a block whose largest magnitude is amax (R43):
    amax * 2^e lies in [128, 256), clamped to [-127, 127] (the range of a
    power-of-two scale byte); an all-zero block takes e = 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)
    e = np.clip(8 - ex, -127, 127)
    return np.where(amax > 0, e, 0).astype(np.int64)


def fp8_quantize(x: np.ndarray, per_row: bool) -> Tuple[np.ndarray, np.ndarray]:
    """Scaled e4m3 values of x and their exponents: x ~= x8 * 2^-e.

    ``per_row``: one exponent per row of a 2-D x, else one for the whole x.
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.abs(x).max(axis=1) if per_row else np.abs(x).max(initial=0.0)
    e = fp8_exponent(amax)
    scaled = np.ldexp(x, e[:, None] if per_row else e)
    return e4m3_round(scaled), e


def fp8_scores(q: np.ndarray, k2: np.ndarray) -> np.ndarray:
    """Scores in log2 units from FP8 operands (R42, R43): q rows and the key
    matrix k2 (already times scale * log2 e) are quantised, multiplied
    exactly, and the scales removed."""
    q8, eq = fp8_quantize(q, per_row=True)
    k8, ek = fp8_quantize(k2, per_row=False)
    return np.ldexp(q8 @ k8.T, -(eq[:, None] + ek))


def attention_fp8(q: np.ndarray, k2: np.ndarray, v: np.ndarray, chunk: int = 2048) -> np.ndarray:
    """O = softmax_2(S) V with S = fp8_scores(q, k2), in fp64 (R42)."""
    v64 = np.asarray(v, dtype=np.float64)
    out = np.empty((q.shape[0], v64.shape[1]), dtype=np.float64)
    q8, eq = fp8_quantize(q, per_row=True)
    k8, ek = fp8_quantize(k2, per_row=False)
    for i in range(0, q.shape[0], chunk):
        s = np.ldexp(q8[i:i + chunk] @ k8.T, -(eq[i:i + chunk, None] + ek))
        s -= s.max(axis=1, keepdims=True)
        e = np.exp2(s)
        out[i:i + chunk] = (e @ v64) / e.sum(axis=1, keepdims=True)
    return out


def fp8_operands(qm: np.ndarray, km: np.ndarray, vm: np.ndarray, scale: float):
    """The stored bf16 operands the FP8 scores start from (R44), from fp32
    means: Q~ rounded to bf16, K~ times the fp32 product of the softmax scale
    and log2(e) (one fp32 rounding) then rounded to bf16, V~ rounded to bf16."""
    kscale = np.float32(np.float32(scale) * np.float32(LOG2E))
    qb = round_bf16_rne(np.asarray(qm, dtype=np.float32))
    kb = round_bf16_rne((np.asarray(km, dtype=np.float32) * kscale).astype(np.float32))
    vb = round_bf16_rne(np.asarray(vm, dtype=np.float32))
    return qb, kb, vb


def unmerge(o: np.ndarray, part: Partition) -> np.ndarray:
    """Copy each merged output row back to every member, at its original index.

    Unmerge inside the blocks and the inverse reorder compose to this one map
    (HTTM page, key design 1 and 2; LiteVGGT page, key design 3; R30).
    """
    return o[part.group_of]


# --------------------------------------------------------------------------
# The whole layer
# --------------------------------------------------------------------------
@dataclass
class HeadIndex:
    q_match: StreamMatch
    k_match: StreamMatch


@dataclass
class Trace:
    """Every intermediate of a layer, for staged comparison."""

    q_match: List[StreamMatch] = field(default_factory=list)
    k_match: List[StreamMatch] = field(default_factory=list)
    delta: Optional[np.ndarray] = None  # [h][N]
    outlier: Optional[np.ndarray] = None  # [h][N]
    q_final_rep: List[np.ndarray] = field(default_factory=list)
    k_rep: List[np.ndarray] = field(default_factory=list)
    out: Optional[np.ndarray] = None


def match_heads(q: np.ndarray, k: np.ndarray, p: Params, heads: Sequence[int], bf16: bool = False) -> Trace:
    """Steps 1-4 for every listed head (head-wise merging, HTTM page, key design 1).

    With the head-shared partition (partition 2) one topology, matched on
    the listed heads' mean key (R37; ``bf16``: the layer's element type),
    serves the queries and keys of every head (R40).
    """
    tr = Trace()
    if p.partition == 2:
        shared = global_match(head_shared_metric(k, bf16), p, p.kv_ratio)
        for _ in heads:
            tr.q_match.append(shared)
            tr.k_match.append(shared)
            tr.k_rep.append(shared.rep)
        return tr
    for i in range(len(heads)):
        if p.partition == 1:  # geometry-aware three-class partition (R31)
            tr.q_match.append(ga_match_stream(q[i], p))
            tr.k_match.append(ga_match_stream(k[i], p))
        else:
            tr.q_match.append(match_stream(q[i], p, p.q_ratio, p.q_dst_stride))
            tr.k_match.append(match_stream(k[i], p, p.kv_ratio, p.kv_dst_stride))
        tr.k_rep.append(tr.k_match[-1].rep)
    return tr


def deviations(q: np.ndarray, q_reps: Sequence[np.ndarray]) -> np.ndarray:
    """delta [h][N] from the initial query partitions (step 5a)."""
    out = np.empty((len(q_reps), q.shape[1]), dtype=np.float32)
    for i, rep in enumerate(q_reps):
        part = partition(rep)
        out[i] = deviation(q[i], part, group_means(q[i], part))
    return out


def head_output(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_final_rep: np.ndarray,
                k_rep: np.ndarray, scale: float, rows: Optional[np.ndarray] = None,
                fp8: bool = False) -> np.ndarray:
    """Steps 6-7 for one head: means, attention, unmerge.

    ``rows`` restricts the output to those original token ids (the attention
    of one output row needs only its own query slot), for large layers.
    ``fp8``: scores from FP8 queries and keys (R41-R44).
    """
    qp = partition(q_final_rep)
    kp = partition(k_rep)
    qt = group_means(q, qp)
    kt = group_means(k, kp)
    vt = group_means(v, kp)
    if fp8:
        qb, kb, vb = fp8_operands(qt, kt, vt, scale)
        if rows is None:
            return unmerge(attention_fp8(qb, kb, vb), qp)
        return attention_fp8(qb[qp.group_of[rows]], kb, vb)
    if rows is None:
        return unmerge(attention(qt, kt, vt, scale), qp)
    slots = qp.group_of[rows]
    return attention(qt[slots], kt, vt, scale)


def layer(q: np.ndarray, k: np.ndarray, v: np.ndarray, p: Params,
          out_heads: Optional[Sequence[int]] = None, rows: Optional[np.ndarray] = None,
          bf16: bool = False) -> Trace:
    """One HTTM global-attention layer (HTTM page, overall framework).

    q, k, v: [h][N][d] fp32 (bf16 inputs upcast exactly).  Steps 1-5 run on
    every head because the outlier budget is shared across heads; steps 6-7
    run for ``out_heads`` (default all) and, if given, only for ``rows``.
    ``bf16``: the layer's element type is bf16 (only the head-shared metric
    of partition 2 depends on it).
    """
    h = q.shape[0]
    tr = match_heads(q, k, p, list(range(h)), bf16=bf16)
    tr.delta = deviations(q, [m.rep for m in tr.q_match])
    tr.outlier = select_outliers(tr.delta, outlier_budget(p))
    tr.q_final_rep = [restore_partition(tr.q_match[i].rep, tr.outlier[i]) for i in range(h)]
    hs = list(range(h)) if out_heads is None else list(out_heads)
    outs = [head_output(q[i], k[i], v[i], tr.q_final_rep[i], tr.k_rep[i], p.scale, rows, p.attn_fp8)
            for i in hs]
    tr.out = np.stack(outs)
    return tr


def layer_cached(q: np.ndarray, k: np.ndarray, v: np.ndarray, p: Params,
                 q_final_rep: Sequence[np.ndarray], k_rep: Sequence[np.ndarray],
                 out_heads: Optional[Sequence[int]] = None,
                 rows: Optional[np.ndarray] = None) -> np.ndarray:
    """A layer that reuses earlier merge indices (LiteVGGT page, key design 3; R22).

    The reordering, the final query partition (outliers already restored) and
    the key partition come from the layer that computed them; only the means
    are recomputed from this layer's q, k, v.
    """
    hs = list(range(q.shape[0])) if out_heads is None else list(out_heads)
    return np.stack([head_output(q[i], k[i], v[i], q_final_rep[i], k_rep[i], p.scale, rows, p.attn_fp8)
                     for i in hs])
