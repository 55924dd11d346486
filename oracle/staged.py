"""Staged comparison of an implementation's intermediates with the oracle.

TEST INFRASTRUCTURE ONLY (see httm_oracle).  The caller passes the other
implementation's intermediates as plain numpy arrays; nothing here imports
or calls that implementation.

Index decisions are compared exactly, except where the oracle itself finds a
near-tie (similarity within 1e-5 of the best, or a source score within 1e-5 of
the r-th score), which is counted.  Every later stage is re-run by the oracle
on the implementation's own indices, so a counted near-tie never cascades:

  (i)   matches and scores, per block (geometry-aware partition: variance
        map and classes exactly, then matches and scores over all
        destinations);
  (ii)  top-r selection and the resulting groups (groups exactly);
  (iii) deviations on the implementation's query groups (bit for bit), and
        the global outlier choice on the implementation's deviations
        (exactly);
  (iv)  final query partition (exactly) and outputs within tolerance.
"""
from __future__ import annotations

import concurrent.futures as cf
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from . import httm_oracle as O

NEAR_TIE = 1e-5


class ParityError(AssertionError):
    pass


def canonical(slot: np.ndarray) -> np.ndarray:
    """Group label -> smallest token id of the group, per token."""
    slot = np.asarray(slot, dtype=np.int64)
    n = np.arange(len(slot))
    u, inv = np.unique(slot, return_inverse=True)
    mins = np.full(len(u), np.iinfo(np.int64).max, dtype=np.int64)
    np.minimum.at(mins, inv, n)
    return mins[inv]


@dataclass
class Report:
    n_src: int = 0
    match_near_ties: int = 0
    select_near_ties: int = 0
    max_score_err: float = 0.0
    delta_nonexact: int = 0
    max_delta_err: float = 0.0
    outlier_threshold_ties: int = 0
    max_out_err: float = 0.0
    out_rms: float = 0.0
    notes: List[str] = field(default_factory=list)

    def as_dict(self) -> Dict:
        return dict(self.__dict__)


def check_stream(x: np.ndarray, p: O.Params, ratio: float, stride: int, gpu_match: np.ndarray,
                 gpu_score: np.ndarray, gpu_group: np.ndarray, rep: Report, what: str) -> np.ndarray:
    """Stages (i)-(ii) for one head and stream; returns the canonical groups.

    gpu_match: destination index (inside its block) per source, sources
    ordered by block then block position; gpu_score: cosine of that match;
    gpu_group: merged slot of every token.
    """
    s = O.dst_stride(ratio, stride)
    N = p.n_tokens
    rep_gpu = canonical(gpu_group)
    label = np.arange(N, dtype=np.int64)  # group built from the implementation's own decisions
    k0 = 0
    for b in O.blocks(p):
        tok = b.tokens
        dpos, spos, sim = O.block_similarity(x[tok], s)
        ns = len(spos)
        gm = np.asarray(gpu_match[k0:k0 + ns], dtype=np.int64)
        gs = np.asarray(gpu_score[k0:k0 + ns], dtype=np.float32)
        k0 += ns
        if ns == 0:
            continue
        if gm.min() < 0 or gm.max() >= len(dpos):
            raise ParityError(f"{what}: match index out of range in block {b.g},{b.a}")
        jo = np.argmax(sim, axis=1)
        rows = np.arange(ns)
        gap = sim[rows, jo] - sim[rows, gm]
        bad = (gm != jo) & (gap >= NEAR_TIE)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise ParityError(f"{what}: block {b.g},{b.a} source {i} matched dst {gm[i]} (sim {sim[i, gm[i]]:.7f})"
                              f" but best is {jo[i]} (sim {sim[i, jo[i]]:.7f})")
        rep.match_near_ties += int(((gm != jo) & (gap < NEAR_TIE)).sum())
        err = np.abs(gs.astype(np.float64) - sim[rows, gm])
        rep.max_score_err = max(rep.max_score_err, float(err.max()))
        if err.max() >= NEAR_TIE:
            raise ParityError(f"{what}: score error {err.max():.3g} in block {b.g},{b.a}")
        # (ii) selection: a source is merged iff it sits in its match's group
        src_tok, dst_tok = tok[spos], tok[dpos[gm]]
        sel = rep_gpu[src_tok] == rep_gpu[dst_tok]
        r = O.merge_count(ratio, b.n, ns)
        if int(sel.sum()) != r:
            raise ParityError(f"{what}: block {b.g},{b.a} merged {int(sel.sum())} sources, expected r={r}")
        so = sim[rows, jo]
        osel = O.select_top_r(so, spos, r)
        if r > 0 and r < ns:
            thr = np.sort(so)[::-1][r - 1]
            diff = sel != osel
            if (diff & (np.abs(so - thr) >= NEAR_TIE)).any():
                i = int(np.flatnonzero(diff & (np.abs(so - thr) >= NEAR_TIE))[0])
                raise ParityError(f"{what}: block {b.g},{b.a} selection differs at source {i} "
                                  f"(score {so[i]:.7f}, r-th {thr:.7f})")
            rep.select_near_ties += int(diff.sum())
        elif (sel != osel).any():
            raise ParityError(f"{what}: block {b.g},{b.a} selection differs with r={r}, |S|={ns}")
        label[src_tok[sel]] = dst_tok[sel]
        rep.n_src += ns
    want = canonical(label)
    if not np.array_equal(want, rep_gpu):
        i = int(np.flatnonzero(want != rep_gpu)[0])
        raise ParityError(f"{what}: groups differ at token {i}: rep {rep_gpu[i]} vs {want[i]}")
    return rep_gpu


def check_ga_stream(x: np.ndarray, p: O.Params, gpu_var: np.ndarray, gpu_role: np.ndarray,
                    gpu_match: np.ndarray, gpu_score: np.ndarray, gpu_group: np.ndarray, rep: Report,
                    what: str, chunk: int = 2048, check_matches: bool = True) -> np.ndarray:
    """Geometry-aware partition of one head and stream; returns the canonical groups.

    (i) the variance map bit for bit; (ii) the three classes bit for bit,
    recomputed from the implementation's own map; (iii) every source's
    destination is the oracle's most similar one or a counted near-tie, its
    score within 1e-5; (iv) groups exactly: each destination with the
    sources that the implementation matched to it.
    gpu_match: matched destination token per token (-1 for non-sources).
    check_matches=False skips the similarity work of (iii) (every match must
    still name a destination, and (iv) still holds).
    """
    N = p.n_tokens
    v = O.token_variance_map(x, p)
    gv = np.asarray(gpu_var, dtype=np.float32)
    if not np.array_equal(v, gv):
        bad = np.flatnonzero(v != gv)
        raise ParityError(f"{what}: variance map differs at {len(bad)} tokens (first {bad[0]}: "
                          f"{gv[bad[0]]!r} vs {v[bad[0]]!r})")
    role = O.ga_roles(gv, p)
    gr = np.asarray(gpu_role, dtype=np.int8)
    if not np.array_equal(role, gr):
        bad = np.flatnonzero(role != gr)
        raise ParityError(f"{what}: classes differ at {len(bad)} tokens (first {bad[0]}: {gr[bad[0]]} vs "
                          f"{role[bad[0]]})")
    src = np.flatnonzero(role == O.ROLE_SRC)
    dst = np.flatnonzero(role == O.ROLE_DST)
    gm = np.asarray(gpu_match, dtype=np.int64)
    if (gm[role != O.ROLE_SRC] != -1).any():
        raise ParityError(f"{what}: a token that is not a source carries a match")
    label = np.arange(N, dtype=np.int64)
    if len(src):
        m = gm[src]
        pos = np.searchsorted(dst, m)
        if (m < 0).any() or (pos >= len(dst)).any() or (dst[np.minimum(pos, len(dst) - 1)] != m).any():
            raise ParityError(f"{what}: a source is matched to a token that is not a destination")
        gs = np.asarray(gpu_score, dtype=np.float32)[src]
        for c0 in range(0, len(src) if check_matches else 0, chunk):
            sc = src[c0:c0 + chunk]
            sim = O.ga_similarity(x, sc, dst)
            rows = np.arange(len(sc))
            jo = np.argmax(sim, axis=1)
            jg = pos[c0:c0 + chunk]
            gap = sim[rows, jo] - sim[rows, jg]
            bad = (jg != jo) & (gap >= NEAR_TIE)
            if bad.any():
                i = int(np.flatnonzero(bad)[0])
                raise ParityError(f"{what}: source {sc[i]} matched {dst[jg[i]]} (sim {sim[i, jg[i]]:.7f}) but "
                                  f"best is {dst[jo[i]]} (sim {sim[i, jo[i]]:.7f})")
            rep.match_near_ties += int(((jg != jo) & (gap < NEAR_TIE)).sum())
            err = np.abs(gs[c0:c0 + chunk].astype(np.float64) - sim[rows, jg])
            rep.max_score_err = max(rep.max_score_err, float(err.max()))
            if err.max() >= NEAR_TIE:
                raise ParityError(f"{what}: score error {err.max():.3g}")
        label[src] = m
        rep.n_src += len(src)
    want = canonical(label)
    got = canonical(gpu_group)
    if not np.array_equal(want, got):
        i = int(np.flatnonzero(want != got)[0])
        raise ParityError(f"{what}: groups differ at token {i}: rep {got[i]} vs {want[i]}")
    return got


def check_gm(k: np.ndarray, p: O.Params, gpu_metric: np.ndarray, gpu_match: np.ndarray, gpu_score: np.ndarray,
             gpu_group: np.ndarray, rep: Report, bf16: bool, chunk: int = 2048) -> np.ndarray:
    """Head-shared global matching; returns the canonical shared groups.

    (i) the head-mean metric bit for bit; (ii) every source's destination is
    the oracle's most similar one or a counted near-tie, its score within
    1e-5; (iii) r sources merged, the merged set equal to the oracle's top-r
    except counted ties within 1e-5 of the r-th score, groups exactly what
    the implementation's own matches and selection imply.
    gpu_metric: [N][d] float; gpu_match: matched destination token per token
    (-1 for non-sources); gpu_group: slot of every token (one head's).
    """
    N = p.n_tokens
    m = O.head_shared_metric(k, bf16)
    gm = np.asarray(gpu_metric, dtype=np.float32)
    if not np.array_equal(m.view(np.uint32), gm.view(np.uint32)):
        bad = np.flatnonzero((m != gm).any(axis=1))
        raise ParityError(f"head-shared metric differs at {len(bad)} tokens (first {bad[0]})")
    tok = np.flatnonzero(~O.is_special(p))
    pos = np.arange(len(tok))
    dpos, spos = pos[pos % O.GM_STRIDE == 0], pos[pos % O.GM_STRIDE != 0]
    src, dst = tok[spos], tok[dpos]
    match = np.asarray(gpu_match, dtype=np.int64)
    if (match[np.setdiff1d(np.arange(N), src)] != -1).any():
        raise ParityError("head-shared: a token that is not a source carries a match")
    rep_gpu = canonical(gpu_group)
    if len(src) == 0:
        if not np.array_equal(rep_gpu, np.arange(N)):
            raise ParityError("head-shared: groups without sources")
        return rep_gpu
    mj = np.searchsorted(dst, match[src])
    if (mj >= len(dst)).any() or (dst[np.minimum(mj, len(dst) - 1)] != match[src]).any():
        raise ParityError("head-shared: a source is matched to a token that is not a destination")
    gs = np.asarray(gpu_score, dtype=np.float32)[src]
    dn = O.row_normalize(m[dst])
    so = np.empty(len(src), dtype=np.float32)
    for c0 in range(0, len(src), chunk):
        sim = (O.row_normalize(m[src[c0:c0 + chunk]]) @ dn.T).astype(np.float32)
        rows = np.arange(sim.shape[0])
        jo = np.argmax(sim, axis=1)
        jg = mj[c0:c0 + chunk]
        gap = sim[rows, jo] - sim[rows, jg]
        bad = (jg != jo) & (gap >= NEAR_TIE)
        if bad.any():
            i = int(np.flatnonzero(bad)[0])
            raise ParityError(f"head-shared: source {src[c0 + i]} matched {dst[jg[i]]} (sim {sim[i, jg[i]]:.7f}) "
                              f"but best is {dst[jo[i]]} (sim {sim[i, jo[i]]:.7f})")
        rep.match_near_ties += int(((jg != jo) & (gap < NEAR_TIE)).sum())
        err = np.abs(gs[c0:c0 + chunk].astype(np.float64) - sim[rows, jg])
        rep.max_score_err = max(rep.max_score_err, float(err.max()))
        if err.max() >= NEAR_TIE:
            raise ParityError(f"head-shared: score error {err.max():.3g}")
        so[c0:c0 + chunk] = sim[rows, jo]
    sel = rep_gpu[src] == rep_gpu[match[src]]
    r = O.merge_count(p.kv_ratio, len(tok), len(src))
    if int(sel.sum()) != r:
        raise ParityError(f"head-shared: {int(sel.sum())} sources merged, expected r={r}")
    osel = O.select_top_r(so, spos, r)
    diff = sel != osel
    if diff.any():
        thr = np.sort(so)[::-1][r - 1] if r > 0 else np.inf
        if (np.abs(so[diff] - thr) >= NEAR_TIE).any():
            raise ParityError("head-shared: merged set differs away from the r-th score")
        rep.select_near_ties += int(diff.sum())
    label = np.arange(N, dtype=np.int64)
    label[src[sel]] = match[src[sel]]
    want = canonical(label)
    if not np.array_equal(want, rep_gpu):
        i = int(np.flatnonzero(want != rep_gpu)[0])
        raise ParityError(f"head-shared: groups differ at token {i}: rep {rep_gpu[i]} vs {want[i]}")
    rep.n_src += len(src)
    return rep_gpu


def check_layer(q: np.ndarray, k: np.ndarray, v: np.ndarray, p: O.Params, gpu: Dict[str, np.ndarray],
                out_gpu: np.ndarray, out_heads: Optional[Sequence[int]] = None,
                rows: Optional[np.ndarray] = None, out_tol: Optional[float] = None,
                match_heads: Optional[Sequence[int]] = None, rel_tol: Optional[float] = None,
                workers: int = 1, out_half_ulp: bool = False, delta_exact: bool = True,
                bf16: bool = False) -> Report:
    """Staged parity of one layer.

    gpu: q_match, q_score, kv_match, kv_score ([h][src]), q_group, kv_group,
    q_slot ([h][N]), delta ([h][N] float32), outlier ([h][N] uint8); under
    the geometry-aware partition ga_var, ga_role, ga_match, ga_score
    ([2][h][N], stream 0 = Q) in place of the four match / score items.
    out_gpu: [h][N][d] as float64/float32.  Tolerance on the max-abs output
    error: ``rel_tol`` * RMS(oracle output) if given (bf16: 2e-2), else
    ``out_tol`` (default 1e-4, fp32).  ``out_half_ulp`` adds half a bf16 ulp
    of the largest reference value (2^-9 * max|ref|), the error that rounding
    the output to bf16 alone can reach: needed where max|ref| exceeds ~2.5 x
    RMS (tiny or heavily merged layers), since there one rounding step of the
    largest outputs is larger than 2e-2 x RMS.  ``workers`` threads share the
    per-head work (numpy releases the GIL in its array kernels).
    Head-shared partition (partition 2): gm_metric ([N][d] float), gm_match,
    gm_score ([N]) in place of the match / score items; ``bf16`` states the
    layer's element type (the metric is rounded to it); every head's query
    and key groups must be the one shared partition.
    ``delta_exact`` (default) requires the deviations bit for bit on the
    implementation's groups (the same fp32 operation sequence); False
    accepts differences within 1e-5 x max(1, delta) and only counts them.
    """
    rep = Report()
    h, N = q.shape[0], q.shape[1]
    mh = list(range(h)) if match_heads is None else list(match_heads)
    q_rep = [None] * h
    k_rep = [None] * h

    ga = p.partition == 1
    if ga:
        ga_items = {it: np.asarray(gpu[it]).reshape(2, h, N) for it in ("ga_var", "ga_role", "ga_match", "ga_score")}
    shared = None
    if p.partition == 2:
        shared = check_gm(k, p, np.asarray(gpu["gm_metric"]).reshape(N, -1), gpu["gm_match"], gpu["gm_score"],
                          gpu["kv_group"][0], rep, bf16)

    def per_head(i):
        r = Report()
        if shared is not None:
            # one partition for the queries and keys of every head
            for nm in ("q_group", "kv_group"):
                if not np.array_equal(canonical(gpu[nm][i]), shared):
                    raise ParityError(f"head {i}: {nm} is not the shared partition")
            return shared, shared, r
        if ga:
            # variance map, classes and groups on every head; the argmax of
            # the matches on the match heads
            qr, kr = (check_ga_stream(x[i], p, ga_items["ga_var"][st, i], ga_items["ga_role"][st, i],
                                      ga_items["ga_match"][st, i], ga_items["ga_score"][st, i],
                                      gpu[grp][i], r, f"head {i} {nm}", check_matches=i in mh)
                      for st, (x, grp, nm) in enumerate(((q, "q_group", "Q"), (k, "kv_group", "K"))))
        elif i in mh:
            qr = check_stream(q[i], p, p.q_ratio, p.q_dst_stride, gpu["q_match"][i], gpu["q_score"][i],
                              gpu["q_group"][i], r, f"head {i} Q")
            kr = check_stream(k[i], p, p.kv_ratio, p.kv_dst_stride, gpu["kv_match"][i],
                              gpu["kv_score"][i], gpu["kv_group"][i], r, f"head {i} K")
        else:
            qr, kr = canonical(gpu["q_group"][i]), canonical(gpu["kv_group"][i])
        return qr, kr, r

    with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        for i, (qr, kr, r) in enumerate(ex.map(per_head, range(h))):
            q_rep[i], k_rep[i] = qr, kr
            rep.n_src += r.n_src
            rep.match_near_ties += r.match_near_ties
            rep.select_near_ties += r.select_near_ties
            rep.max_score_err = max(rep.max_score_err, r.max_score_err)
    # (iii) deviations on the implementation's query groups
    with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        delta_o = np.stack(list(ex.map(lambda i: O.deviations(q[i:i + 1], [q_rep[i]])[0], range(h))))
    dg = gpu["delta"].astype(np.float32)
    rep.delta_nonexact = int((dg != delta_o).sum())
    rep.max_delta_err = float(np.abs(dg.astype(np.float64) - delta_o).max())
    if delta_exact and rep.delta_nonexact:
        h0, n0 = (int(a[0]) for a in np.nonzero(dg != delta_o))
        raise ParityError(f"deviation differs at {rep.delta_nonexact} tokens (first head {h0} token {n0}: "
                          f"{dg[h0, n0]!r} vs {delta_o[h0, n0]!r})")
    tol = NEAR_TIE * np.maximum(1.0, delta_o)
    if (np.abs(dg.astype(np.float64) - delta_o) > tol).any():
        raise ParityError(f"deviation error {rep.max_delta_err:.3g}")
    k_o = O.outlier_budget(p)
    mask_gpu = gpu["outlier"].astype(bool)
    if not np.array_equal(O.select_outliers(dg, k_o), mask_gpu):
        raise ParityError("outlier mask differs from the global top-k_o of the implementation's deviations")
    mo = O.select_outliers(delta_o, k_o)
    if not np.array_equal(mo, mask_gpu):
        flat = np.sort(delta_o.reshape(-1))[::-1]
        thr = flat[k_o - 1] if k_o > 0 else np.inf
        diff = mo != mask_gpu
        if (np.abs(delta_o[diff] - thr) > NEAR_TIE * max(1.0, thr)).any():
            raise ParityError("outlier mask differs away from the threshold")
        rep.outlier_threshold_ties = int(diff.sum())
    # (iv) final query partition and outputs
    qf = []
    for i in range(h):
        want = O.restore_partition(q_rep[i], mask_gpu[i])
        got = canonical(gpu["q_slot"][i])
        if not np.array_equal(want, got):
            j = int(np.flatnonzero(want != got)[0])
            raise ParityError(f"head {i}: final query partition differs at token {j}")
        qf.append(got)
    hs = list(range(h)) if out_heads is None else list(out_heads)
    outs = []
    for i in hs:
        outs.append(O.head_output(q[i], k[i], v[i], qf[i], k_rep[i], p.scale, rows, p.attn_fp8))
    ref = np.stack(outs)
    got = out_gpu[hs] if rows is None else out_gpu[hs][:, rows]
    rep.out_rms = float(np.sqrt(np.mean(ref ** 2)))
    rep.max_out_err = float(np.abs(got.astype(np.float64) - ref).max())
    if rel_tol is not None:
        out_tol = rel_tol * rep.out_rms
    elif out_tol is None:
        out_tol = 1e-4
    if out_half_ulp:
        out_tol += 2.0 ** -9 * float(np.abs(ref).max())
    if not rep.max_out_err <= out_tol:
        raise ParityError(f"output error {rep.max_out_err:.3g} > {out_tol:.3g} (rms {rep.out_rms:.3g})")
    return rep
