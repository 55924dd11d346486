"""A layer call enqueues only kernels and event waits (no allocation, no
memset), so it can be captured in a HIP graph.  Every replay, with the
program's own eager layers and synchronizations in between, must give the
eager result bit for bit, for both partitions and for cached layers."""
import numpy as np
import pytest
import torch

import gen
import token_merged_global_amd as H

from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _small(partition, fp8=False):
    w = gen.WORKLOADS["vggt30"].with_(name="small", cfg_id=7, frames=4, heads=3, n_t=2, attn_fp8=fp8)
    return w.with_(partition=1, protect_pct=10.0) if partition else w


@pytest.mark.parametrize("partition,fp8", [(0, False), (1, False), (0, True)])
def test_graph_replays_match_eager(partition, fp8):
    w = _small(partition, fp8)
    x = gen.layer_inputs(w)
    x2 = gen.layer_inputs(w, seed=gen.DEFAULT_SEED + 9)
    plan = H.Plan.from_workload(w)
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    q2, k2, v2 = (to_dev(x2[t], w.dtype) for t in "qkv")
    ws, ws2 = H.workspace(plan), H.workspace(plan)
    out, out2 = torch.empty_like(q), torch.empty_like(q)
    idx = H.CachedIndex(plan)
    eager = H.layer(plan, q, k, v, ws=ws, out=out, index=idx).clone()
    eager_c = H.layer_cached(plan, idx, q2, k2, v2, ws=ws).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm call on the capture stream
        H.layer(plan, q, k, v, ws=ws, out=out, index=idx)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    oc = torch.empty_like(q)
    with torch.cuda.graph(g):
        H.layer(plan, q, k, v, ws=ws, out=out, index=idx)
        H.layer_cached(plan, idx, q2, k2, v2, ws=ws, out=oc)
    for rep in range(4):
        out.zero_()
        oc.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), rep
        assert torch.equal(oc.view(torch.int16), eager_c.view(torch.int16)), rep
        # the program's own eager work between replays, on other buffers
        H.layer(plan, q2, k2, v2, ws=ws2, out=out2)
        torch.cuda.synchronize()
    say(f"[graph partition {partition} fp8 {fp8}] 4 replays equal to eager")
