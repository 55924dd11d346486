"""CPU checks of the staged checker's geometry-aware stages: the oracle's own
intermediates pass, and a planted mistake in any stage is caught."""
import numpy as np
import pytest

import gen
import oracle as O
from oracle import staged


def _case():
    w = gen.Workload(name="ga_chk", cfg_id=13, dtype="f32", heads=2, d_head=64, frames=4, grid_h=5, grid_w=6,
                     n_special=1, n_s=8, n_t=2, q_ratio=0.5, kv_ratio=0.5, outlier_pct=10.0, partition=1,
                     protect_pct=10.0)
    x = gen.layer_inputs(w)
    p = O.Params.from_workload(w)
    return w, x, p


def _fake_gpu(x, p):
    """The intermediates an implementation hands to the checker, from the oracle."""
    h, N = x["q"].shape[:2]
    gpu = {k: np.zeros((2, h, N), dtype=dt) for k, dt in
           (("ga_var", np.float32), ("ga_role", np.uint8), ("ga_match", np.int32), ("ga_score", np.float32))}
    reps = {}
    for st, t in enumerate("qk"):
        for i in range(h):
            v = O.token_variance_map(x[t][i], p)
            m = O.ga_match_stream(x[t][i], p)
            gpu["ga_var"][st, i] = v
            gpu["ga_role"][st, i] = O.ga_roles(v, p)
            gpu["ga_match"][st, i] = np.where(m.is_src, m.match_dst, -1)
            gpu["ga_score"][st, i] = np.where(m.is_src, m.score, 0.0)
            reps[(t, i)] = m.rep
    gpu["q_group"] = np.stack([reps[("q", i)] for i in range(h)])
    gpu["kv_group"] = np.stack([reps[("k", i)] for i in range(h)])
    delta = O.deviations(x["q"], [reps[("q", i)] for i in range(h)])
    mask = O.select_outliers(delta, O.outlier_budget(p))
    gpu["delta"] = delta
    gpu["outlier"] = mask.astype(np.uint8)
    gpu["q_slot"] = np.stack([O.restore_partition(reps[("q", i)], mask[i]) for i in range(h)])
    return gpu


def test_oracle_intermediates_pass():
    w, x, p = _case()
    gpu = _fake_gpu(x, p)
    tr = O.layer(x["q"], x["k"], x["v"], p)
    rep = staged.check_layer(x["q"], x["k"], x["v"], p, gpu, tr.out, out_tol=1e-6)
    assert rep.n_src > 0 and rep.match_near_ties == 0 and rep.delta_nonexact == 0


@pytest.mark.parametrize("what", ["var", "role", "match", "score", "group"])
def test_planted_mistakes_are_caught(what):
    w, x, p = _case()
    gpu = _fake_gpu(x, p)
    tr = O.layer(x["q"], x["k"], x["v"], p)
    src = np.flatnonzero(gpu["ga_role"][1, 0] == O.ROLE_SRC)
    dst = np.flatnonzero(gpu["ga_role"][1, 0] == O.ROLE_DST)
    s = src[len(src) // 2]
    if what == "var":  # one ulp on one patch token
        j = w.n_special + 3
        gpu["ga_var"][1, 0, j] = np.nextafter(gpu["ga_var"][1, 0, j], np.float32(np.inf))
    elif what == "role":  # a source relabelled as a destination
        gpu["ga_role"][1, 0, s] = O.ROLE_DST
    elif what == "match":  # the least similar destination instead of the best
        sim = O.ga_similarity(x["k"][0], np.array([s]), dst)[0]
        gpu["ga_match"][1, 0, s] = dst[int(np.argmin(sim))]
    elif what == "score":
        gpu["ga_score"][1, 0, s] += np.float32(1e-3)
    elif what == "group":  # a source left alone although it has a match
        g = gpu["kv_group"][0].copy()
        g[s] = w.n_tokens + 7
        gpu["kv_group"] = np.stack([g, gpu["kv_group"][1]])
    with pytest.raises(staged.ParityError):
        staged.check_layer(x["q"], x["k"], x["v"], p, gpu, tr.out, out_tol=1e-6)
