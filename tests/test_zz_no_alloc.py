"""The allocation-free layer entry point (httm_layer_noalloc) against the
layer with a caller workspace (httm_layer), through the C ABI: two calls in a
row, the second on a smaller layer, each bit-identical to httm_layer on the
same inputs (the same kernels run, one stream instead of two); a plan whose
workspace exceeds the static scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import gen
import token_merged_global_amd as H
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _small(frames, heads, n_t, **kw):
    return gen.WORKLOADS["vggt30"].with_(name="small", cfg_id=7, frames=frames, heads=heads, n_t=n_t, **kw)


def _pair(w, seed):
    x = gen.layer_inputs(w, seed=seed)
    plan = H.Plan.from_workload(w)
    assert plan.workspace_bytes <= H.noalloc_capacity()
    q, k, v = (to_dev(x[t], w.dtype) for t in "qkv")
    ref = H.layer(plan, q, k, v, ws=H.workspace(plan))
    out = torch.empty_like(q)
    H.layer_noalloc(plan, q, k, v, out)
    torch.cuda.synchronize()
    bits = torch.int16 if w.dtype == "bf16" else torch.int32
    same = torch.equal(out.view(bits), ref.view(bits))
    say(f"[noalloc] {w.name} {w.dtype} N={w.n_tokens} heads={w.heads}: bit-identical={same}")
    assert same
    return out


def test_noalloc_matches_layer_two_calls_second_smaller():
    assert H.noalloc_capacity() == 64 << 20
    _pair(_small(6, 4, 3), gen.DEFAULT_SEED)       # 8,244 tokens x 4 heads
    _pair(_small(4, 2, 2), gen.DEFAULT_SEED + 1)   # then a smaller layer: 5,496 tokens x 2 heads
    _pair(gen.WORKLOADS["tiny"], gen.DEFAULT_SEED)  # and the fp32 layer
    _pair(_small(4, 2, 2, attn_fp8=True), gen.DEFAULT_SEED)  # and FP8 scores


def test_noalloc_refuses_a_layer_beyond_its_scratch():
    w = gen.WORKLOADS["vggt30"]
    plan = H.Plan.from_workload(w)
    assert plan.workspace_bytes > H.noalloc_capacity()
    q = torch.zeros((w.heads, w.n_tokens, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(H.HttmError) as e:
        H.layer_noalloc(plan, q, q, q, torch.empty_like(q))
    assert e.value.status == 3 and "httm_layer_noalloc holds" in str(e.value)
