"""CPU checks of the staged checker's head-shared stage (partition 2): the
oracle's own intermediates pass; a planted mistake in the metric, a match, a
score, the merged set or one head's groups is caught."""
import numpy as np
import pytest

import gen
import oracle as O
from oracle import staged


def _case():
    w = gen.Workload(name="gm_chk", cfg_id=15, dtype="f32", heads=3, d_head=64, frames=4, grid_h=5, grid_w=6,
                     n_special=1, n_s=8, n_t=2, q_ratio=0.5, kv_ratio=0.5, outlier_pct=10.0, partition=2)
    x = gen.layer_inputs(w)
    return w, x, O.Params.from_workload(w)


def _fake_gpu(x, p):
    h, N = x["q"].shape[:2]
    m = O.head_shared_metric(x["k"], False)
    g = O.global_match(m, p, p.kv_ratio)
    gpu = {"gm_metric": m.copy(), "gm_match": np.where(g.is_src, g.match_dst, -1).astype(np.int32),
           "gm_score": np.where(g.is_src, g.score, 0.0).astype(np.float32),
           "q_group": np.stack([g.rep] * h), "kv_group": np.stack([g.rep] * h)}
    delta = O.deviations(x["q"], [g.rep] * h)
    mask = O.select_outliers(delta, O.outlier_budget(p))
    gpu["delta"] = delta
    gpu["outlier"] = mask.astype(np.uint8)
    gpu["q_slot"] = np.stack([O.restore_partition(g.rep, mask[i]) for i in range(h)])
    return gpu, g


def test_oracle_intermediates_pass():
    w, x, p = _case()
    gpu, _ = _fake_gpu(x, p)
    tr = O.layer(x["q"], x["k"], x["v"], p)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, tr.out, out_tol=1e-6)
    assert rep.n_src > 0 and rep.match_near_ties == 0 and rep.select_near_ties == 0


@pytest.mark.parametrize("what", ["metric", "match", "score", "selection", "head_group"])
def test_planted_mistakes_are_caught(what):
    w, x, p = _case()
    gpu, g = _fake_gpu(x, p)
    tr = O.layer(x["q"], x["k"], x["v"], p)
    src = np.flatnonzero(g.is_src)
    if what == "metric":  # one ulp on one channel of one patch token
        j = w.n_special + 2
        gpu["gm_metric"][j, 5] = np.nextafter(gpu["gm_metric"][j, 5], np.float32(np.inf))
    elif what == "match":  # a source matched to its least similar destination
        tok = np.flatnonzero(~O.is_special(p))
        dst = tok[np.arange(len(tok)) % 4 == 0]
        s = src[len(src) // 3]
        sim = (O.row_normalize(gpu["gm_metric"][[s]]) @ O.row_normalize(gpu["gm_metric"][dst]).T)[0]
        gpu["gm_match"][s] = dst[int(np.argmin(sim))]
    elif what == "score":
        gpu["gm_score"][src[5]] += np.float32(1e-3)
    elif what == "selection":  # the best merged source leaves, the worst unmerged one joins its match
        sel = src[g.selected[src]]
        uns = src[~g.selected[src]]
        best = sel[np.argmax(g.score[sel])]
        worst = uns[np.argmin(g.score[uns])]
        rep = g.rep.copy()
        rep[best] = best
        rep[worst] = rep[g.match_dst[worst]]
        gpu["q_group"] = np.stack([rep] * p.heads)
        gpu["kv_group"] = np.stack([rep] * p.heads)
    elif what == "head_group":  # one head's keys grouped differently
        kg = gpu["kv_group"].copy()
        s = src[g.selected[src]][0]
        kg[2, s] = s
        gpu["kv_group"] = kg
    with pytest.raises(staged.ParityError):
        staged.check_layer(x["q"], x["k"], x["v"], p, gpu, tr.out, out_tol=1e-6)
