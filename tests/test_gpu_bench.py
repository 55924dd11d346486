"""bench.py's output contract on a GPU: one JSON line with the metric, the
whole-job value, the dominant kernel's roofline (achieved / peak from the
live launch timing) and the oracle's CPU baseline, for both partitions.
Run on the small 4-frame workload so that it takes seconds."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                        "--warmup", "1", "--dense-reps", "0", "--cached-layers", "0", "--no-extra", *args],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.parametrize("partition", ["httm", "ga", "global"])
def test_bench_json_contract(partition):
    d = _bench("--partition", partition)
    for key in ["metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"]:
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None
    assert isinstance(d["config"]["workload"], str) and d["config"]["tokens"] > 0
    # whole-job throughput: tokens of the step's layers per step time
    assert d["config"]["layers_per_step"] == 1
    assert d["value"] == pytest.approx(d["config"]["tokens"] / (d["ms_per_step"] * 1e-3), rel=1e-9)
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s"
    assert rf["avg_launch_ms"] > 0 and rf["launches_timed"] == 3
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    if partition == "global":
        assert d["config"]["partition"] == "head-shared global"
        assert d["head_shared"]["match_flop"] > 0
    if partition == "ga":
        assert d["config"]["partition"] == "geometry-aware"
        assert d["geometry_aware"]["match_flop"] > 0
        kernels = {rf["kernel"], d["roofline_other_kernel"]["kernel"]}
        assert any(k.startswith("ga_match") for k in kernels) and any(k.startswith("attn") for k in kernels)
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    mp = d["measured_peaks"]
    assert mp["mfma_bf16"]["achieved"] > 0 and mp["hbm_copy"]["achieved"] > 0
    assert mp["mfma_bf16"]["flop_per_launch"] == 2048 * 120000 * 524288
    assert mp["mfma_fp8"]["achieved"] > 0
    assert mp["mfma_fp8"]["flop_per_launch"] == 2048 * 40000 * 4 * 4 * (2 * 32 * 32 * 64)
    for key, r in d["rooflines"].items():
        assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-9), key
        assert r["bound"] in ("hbm", "mfma"), key
        if r["bound"] == "hbm":
            assert r["frac_measured_peak"] == pytest.approx(r["achieved"] / mp["hbm_copy"]["achieved"], rel=1e-9)


def test_bench_cached_stack_contract():
    """A stack step (layer 0 + cached layers on their own inputs): the value is
    the aggregate throughput of all layers of the step."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3",
                        "--warmup", "1", "--dense-reps", "1", "--cached-layers", "2", "--no-extra"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["config"]["layers_per_step"] == 3
    assert d["value"] == pytest.approx(3 * d["config"]["tokens"] / (d["ms_per_step"] * 1e-3), rel=1e-9)
    st = d["stack"]
    assert st["cached_layers"] == 2 and st["layer0_ms"] > 0 and st["cached_ms_per_layer"] > 0
    assert "merge_q_cached" in d["rooflines"]
    assert d["speedup_vs_unmerged_attention"] > 0


def test_bench_compare_matching():
    """--compare-matching: matching and aggregation of the block-local layer
    against the head-shared global layer on the same inputs."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--compare-matching"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("httm_block_local", "head_shared_global"):
        assert d[key]["matching_ms"] > 0 and d[key]["aggregation_ms"] > 0 and d[key]["layer_ms"] > 0
    assert d["matching_cost_ratio"] > 0 and d["matching_flop_ratio"] > 0
