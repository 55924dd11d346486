"""Host-side checks of the C ABI (no GPU needed, no compute calls).

* libhttm.so loads and exports every function ``include/httm.h`` declares;
* the host plan's block table, strides, merge counts and sizes equal the
  oracle's independent construction (temporal reordering of the HTTM page,
  key design 2; counts of key design 1 / settings);
* validation returns the documented status codes.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import gen
import oracle as O
import token_merged_global_amd as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "httm.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(httm_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = _declared()
    assert len(names) >= 15
    L = H.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in H.EXPORTS, n


def _enum_names(typedef: str, prefix: str):
    """Member names of one `typedef enum { ... } <typedef>;` of the header, in order, without COUNT."""
    txt = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "httm.h")).read(), flags=re.S)
    body = re.search(r"typedef enum \{([^}]*)\}\s*" + typedef + r"\s*;", txt).group(1)
    names = [m.split("=")[0].strip() for m in body.split(",") if m.strip()]
    assert names[-1] == prefix + "COUNT"
    return [n[len(prefix):].lower() for n in names[:-1]]


def test_binding_name_lists_follow_the_header_enums():
    # the binding indexes the library's tables by position in these lists
    assert H.TIMING_STAGES == _enum_names("httm_timing_stage", "HTTM_T_")
    assert H.DEBUG_ITEMS == _enum_names("httm_debug_item", "HTTM_DBG_")


def _plans():
    for name in ["tiny", "vggt30", "vggt100", "vggt200", "vggt500"]:
        yield name, gen.WORKLOADS[name]
    w = gen.WORKLOADS["vggt200"]
    yield "vggt200_kv75", w.with_(kv_ratio=0.75)
    yield "vggt200_ratio0", w.with_(q_ratio=0.0, kv_ratio=0.0)
    yield "odd", gen.Workload(name="odd", cfg_id=9, dtype="bf16", heads=3, d_head=64, frames=7, grid_h=5,
                              grid_w=9, n_special=2, n_s=10, n_t=3, q_ratio=0.6, kv_ratio=0.3,
                              outlier_pct=7.5)
    yield "odd_frame_minor", gen.Workload(name="odd", cfg_id=9, dtype="bf16", heads=3, d_head=64, frames=7,
                                          grid_h=5, grid_w=9, n_special=2, n_s=10, n_t=3, q_ratio=0.6,
                                          kv_ratio=0.3, outlier_pct=7.5, block_order=1)


@pytest.mark.parametrize("name,w", list(_plans()))
def test_plan_matches_oracle_blocks(name, w):
    plan = H.Plan.from_workload(w)
    p = O.Params.from_workload(w)
    ob = O.blocks(p)
    hb = plan.blocks()
    assert len(hb) == len(ob) == plan.info["n_blocks"]
    sq, sk = O.dst_stride(p.q_ratio), O.dst_stride(p.kv_ratio)
    assert (plan.info["q_stride"], plan.info["kv_stride"]) == (sq, sk)
    pi = O.reorder_permutation(p)
    start = 0
    slots = [0, 0]
    srcs = [0, 0]
    for b, (o, h) in enumerate(zip(ob, hb)):
        assert h["start"] == start and h["n"] == o.n
        assert (h["f0"], h["nf"], h["j0"], h["run"]) == (o.f0, o.nf, o.j0, o.run)
        # block position -> token, as the kernels compute it
        i = np.arange(o.n)
        if p.block_order == 0:
            tok = (h["f0"] + i // h["run"]) * p.tokens_per_frame + p.n_special + h["j0"] + i % h["run"]
        else:
            tok = (h["f0"] + i % h["nf"]) * p.tokens_per_frame + p.n_special + h["j0"] + i // h["nf"]
        assert np.array_equal(tok, pi[start:start + o.n])
        for st, (s, ratio, pre) in enumerate([(sq, p.q_ratio, "q"), (sk, p.kv_ratio, "kv")]):
            nd = -(-o.n // s)
            assert h[f"{pre}_dst"] == nd and h[f"{pre}_src"] == o.n - nd
            assert h[f"{pre}_r"] == O.merge_count(ratio, o.n, o.n - nd)
            assert h[f"{pre}_slot0"] == slots[st] and h[f"{pre}_src0"] == srcs[st]
            slots[st] += o.n - h[f"{pre}_r"]
            srcs[st] += o.n - nd
        start += o.n
    spec = p.frames * p.n_special
    assert plan.info["q_groups"] == slots[0] + spec
    assert plan.info["kv_len"] == slots[1] + spec
    assert plan.info["n_outliers"] == O.outlier_budget(p)
    assert plan.info["q_capacity"] == p.heads * plan.info["q_groups"] + O.outlier_budget(p)
    assert plan.info["n_tokens"] == p.n_tokens


def test_vggt30_sizes():
    plan = H.Plan.from_workload(gen.WORKLOADS["vggt30"])
    assert (plan.info["q_groups"], plan.info["kv_len"], plan.info["n_outliers"]) == (4257, 20685, 65952)
    assert abs(plan.info["softmax_scale"] - 0.125) < 1e-9


def _status(**kw):
    base = dict(heads=2, frames=4, grid_h=4, grid_w=4, n_special=1, n_s=8, n_t=2, q_ratio=0.5, kv_ratio=0.5,
                outlier_pct=10.0, dtype="bf16")
    base.update(kw)
    try:
        H.Plan(**base)
        return 0
    except H.HttmError as e:
        return e.status


def test_validation_codes():
    assert _status() == 0
    assert _status(q_ratio=1.0) == 1
    assert _status(kv_ratio=-0.1) == 1
    assert _status(outlier_pct=100.5) == 1
    assert _status(heads=0) == 1
    assert _status(q_dst_stride=1) == 1
    assert _status(d_head=128) == 2
    assert _status(block_order=1) == 0
    assert _status(block_order=2) == 1
    assert _status(n_s=128, n_t=33) == 2  # block larger than 4096
    assert _status(heads=64) == 0
    assert _status(heads=65) == 2  # per-head prefix tables are sized for 64
    # one head of 2^24 tokens: 32-bit offsets into a head's merged keys
    assert _status(heads=1, frames=4096, grid_h=64, grid_w=64, n_special=0, n_s=64, n_t=1) == 2
    assert _status(heads=1, frames=4095, grid_h=64, grid_w=64, n_special=0, n_s=64, n_t=1) == 0
    assert _status(softmax_scale=float("inf")) == 1
    for split in (0, 1, 2, 4, 8):
        assert _status(attn_split=split) == 0
    for split in (-1, 3, 16):
        assert _status(attn_split=split) == 1
    assert _status(partition=2) == 0
    assert _status(partition=3) == 1
    assert _status(attn_fp8=True) == 0
    for part in (1, 2):
        assert _status(attn_fp8=True, partition=part) == 0


def test_fp8_plan_validation_sizes_and_items():
    """FP8 scores: bf16 layers only; the workspace grows by the e4m3 keys
    ([h][L_k padded][64] bytes), the e4m3 queries ([q_capacity][64] bytes),
    their exponents and the key maxima; the FP8 debug items exist only then."""
    w = gen.WORKLOADS["tiny"]  # fp32 layer
    with pytest.raises(H.HttmError) as e:
        H.Plan.from_workload(w, attn_fp8=True)
    assert e.value.status == 2
    w30 = gen.WORKLOADS["vggt30"]
    plan16 = H.Plan.from_workload(w30)
    plan8 = H.Plan.from_workload(w30, attn_fp8=True)
    h, lkp, qc = w30.heads, -(-plan8.info["kv_len"] // 64) * 64, plan8.info["q_capacity"]
    extra = plan8.workspace_bytes - plan16.workspace_bytes
    need = h * lkp * 64 + qc * 64 + 4 * qc + 4 * h + 4 * h * 64
    assert need <= extra <= need + 5 * 256
    assert plan8.index_bytes == plan16.index_bytes
    assert set(H.FP8_ITEMS) <= set(H.debug_items(plan8, rows=True))
    assert not set(H.FP8_ITEMS) & set(H.debug_items(plan16, rows=True))
    n = ctypes.c_size_t()
    assert H.lib().httm_debug_size(plan16.handle, H.DEBUG_ITEMS.index("k8"), ctypes.byref(n)) == 2
    assert H.lib().httm_debug_size(plan8.handle, H.DEBUG_ITEMS.index("k8"), ctypes.byref(n)) == 0
    assert n.value == h * lkp * 64


@pytest.mark.parametrize("name,kv", [("tiny", 0.5), ("vggt30", 0.5), ("vggt30", 0.75), ("vggt500", 0.5)])
def test_head_shared_plan_sizes(name, kv):
    """partition 2: one block of every patch, every 4th a destination, r =
    min(|S|, floor(kv * P)) merged: N - r groups for queries and keys."""
    w = gen.WORKLOADS[name].with_(partition=2, kv_ratio=kv)
    plan = H.Plan.from_workload(w)
    P = w.frames * w.grid_h * w.grid_w
    nd = -(-P // 4)
    r = min(P - nd, int(math.floor(kv * P + 1e-9)))
    assert plan.info["q_groups"] == plan.info["kv_len"] == w.n_tokens - r
    assert plan.info["q_src"] == plan.info["kv_src"] == P - nd
    p = O.Params.from_workload(w)
    if name == "tiny":
        q, k, v = (x for x in (np.random.default_rng(1).standard_normal((1, w.n_tokens, 64)).astype(np.float32),) * 3)
        g = O.global_match(O.head_shared_metric(k, False), p, kv)
        assert len(np.unique(g.rep)) == w.n_tokens - r


def test_layer_rejects_bad_buffers_before_any_launch():
    """Host validation paths (no device call is reached)."""
    L = H.lib()
    plan = H.Plan(heads=1, frames=2, grid_h=4, grid_w=4, n_special=0, n_s=8, n_t=2, q_ratio=0.5,
                  kv_ratio=0.5, outlier_pct=10.0, dtype="f32")
    ws = plan.workspace_bytes
    fake = 1 << 20  # never dereferenced: validation fails first
    st = L.httm_layer(plan.handle, fake, ws - 1, fake, fake, fake, fake, None, None)
    assert st == 3
    st = L.httm_layer(plan.handle, fake, ws, None, fake, fake, fake, None, None)
    assert st == 1
    st = L.httm_layer(plan.handle, fake + 4, ws, fake, fake, fake, fake, None, None)
    assert st == 1
    idx = H.Index(0, fake, plan.index_bytes, 0)
    st = L.httm_layer_cached(plan.handle, fake, ws, ctypes.byref(idx), fake, fake, fake, fake, None)
    assert st == 4
    other = H.Plan(heads=1, frames=2, grid_h=4, grid_w=4, n_special=0, n_s=8, n_t=2, q_ratio=0.5,
                   kv_ratio=0.5, outlier_pct=10.0, dtype="f32")
    idx2 = H.Index(other.handle.value or 0, fake, plan.index_bytes, 1)
    st = L.httm_layer_cached(plan.handle, fake, ws, ctypes.byref(idx2), fake, fake, fake, fake, None)
    assert st == 4
    small = H.Index(0, fake, plan.index_bytes - 1, 0)
    st = L.httm_layer(plan.handle, fake, ws, fake, fake, fake, fake, ctypes.byref(small), None)
    assert st == 3
    assert L.httm_status_string(4).decode().startswith("index")
    n = ctypes.c_size_t()
    assert L.httm_debug_size(plan.handle, 99, ctypes.byref(n)) == 1
    assert L.httm_debug_size(plan.handle, 10, ctypes.byref(n)) == 0 and n.value == 16
    assert L.httm_debug_size(plan.handle, 11, ctypes.byref(n)) == 0 and n.value == 4


def test_index_export_import_validation():
    """Index export/import refuse foreign or malformed bytes before any copy
    (status codes of include/httm.h; the fake device pointer is never used)."""
    plan = H.Plan.from_workload(gen.WORKLOADS["tiny"])
    L = H.lib()
    n = plan.index_bytes
    fake = H.Index(0, 0x1000, n, 0)
    buf = np.zeros(n, dtype=np.uint8)
    # an index this plan did not fill
    assert L.httm_index_export(plan.handle, ctypes.byref(fake), buf.ctypes.data, n, None) == 4
    # NULL arguments
    assert L.httm_index_export(plan.handle, ctypes.byref(fake), None, n, None) == 1
    assert L.httm_index_import(plan.handle, None, n, ctypes.byref(fake), None) == 1
    # wrong size, then the right size with no valid header
    assert L.httm_index_import(plan.handle, buf.ctypes.data, n - 4, ctypes.byref(fake), None) == 4
    assert L.httm_index_import(plan.handle, buf.ctypes.data, n, ctypes.byref(fake), None) == 4
    assert fake.valid == 0
    # a device buffer smaller than the index
    small = H.Index(0, 0x1000, n - 1, 0)
    assert L.httm_index_import(plan.handle, buf.ctypes.data, n, ctypes.byref(small), None) == 3


def _ga_bound(w, pct):
    hw = w.grid_h * w.grid_w
    kp = math.floor(pct / 100.0 * hw + 1e-9)
    cells = ((w.grid_h + 1) // 2) * ((w.grid_w + 1) // 2)
    return min(w.n_tokens, w.frames * w.n_special + hw + (w.frames - 1) * (kp + cells))


@pytest.mark.parametrize("name,pct", [("tiny", 10.0), ("vggt30", 10.0), ("vggt100", 10.0), ("vggt500", 10.0),
                                      ("vggt30", 0.0), ("vggt30", 100.0)])
def test_ga_plan_sizes(name, pct):
    """Geometry-aware plans size every head for the largest possible group
    count: all first-frame patches, specials, and per later frame the
    protected patches plus one destination per 2x2 cell."""
    w = gen.WORKLOADS[name].with_(partition=1, protect_pct=pct)
    plan = H.Plan.from_workload(w)
    b = _ga_bound(w, pct)
    assert plan.info["q_groups"] == plan.info["kv_len"] == b
    assert plan.info["q_capacity"] == w.heads * b + plan.info["n_outliers"]
    assert plan.info["q_src"] == plan.info["kv_src"] == (w.frames - 1) * w.grid_h * w.grid_w
    assert "ga_var" in H.debug_items(plan) and "q_match" not in H.debug_items(plan)
    n = ctypes.c_size_t()
    L = H.lib()
    assert L.httm_debug_size(plan.handle, H.DEBUG_ITEMS.index("q_match"), ctypes.byref(n)) == 2
    assert L.httm_debug_size(plan.handle, H.DEBUG_ITEMS.index("ga_role"), ctypes.byref(n)) == 0
    assert n.value == 2 * w.heads * w.n_tokens
    blk = H.Plan.from_workload(gen.WORKLOADS[name])
    assert L.httm_debug_size(blk.handle, H.DEBUG_ITEMS.index("ga_var"), ctypes.byref(n)) == 2
    # the index differs from the block-local plan's: another layout, another fingerprint
    assert plan.index_bytes > 0


def test_ga_group_bound_holds_on_the_oracle():
    """The plan's bound is never exceeded by the oracle's groups, with
    protected cells and odd grid edges."""
    for gh, gw, pct, sp in [(5, 7, 20.0, 2), (4, 4, 0.0, 0), (3, 5, 60.0, 1)]:
        w = gen.Workload(name="ga", cfg_id=11, dtype="f32", heads=2, d_head=64, frames=5, grid_h=gh, grid_w=gw,
                         n_special=sp, n_s=8, n_t=2, q_ratio=0.5, kv_ratio=0.5, outlier_pct=10.0, partition=1,
                         protect_pct=pct)
        p = O.Params.from_workload(w)
        x = gen.layer_inputs(w)
        for t in "qk":
            for hh in range(w.heads):
                m = O.ga_match_stream(x[t][hh], p)
                assert len(np.unique(m.rep)) <= _ga_bound(w, pct)


def test_ga_validation_codes():
    assert _status(partition=1) == 0
    assert _status(partition=3) == 1
    assert _status(partition=-1) == 1
    assert _status(partition=1, protect_pct=-1.0) == 1
    assert _status(partition=1, protect_pct=100.5) == 1
    assert _status(partition=1, protect_pct=float("nan")) == 1
    assert _status(partition=0, protect_pct=-1.0) == 0  # ignored by the block partition
    assert _status(partition=1, grid_h=64, grid_w=64) == 0
    assert _status(partition=1, grid_h=64, grid_w=65) == 2  # more than 4096 patches per frame
    # N = 1000 * 1374 >= 2^20 tokens
    assert _status(partition=1, frames=1000, grid_h=37, grid_w=37, n_special=5, n_s=128, n_t=30) == 2
    assert _status(partition=1, frames=500, grid_h=37, grid_w=37, n_special=5, n_s=128, n_t=30) == 0


def _no_gpu():
    import torch
    return not torch.cuda.is_available()


@pytest.mark.skipif(not _no_gpu(), reason="checks the error path of a host without a GPU")
def test_device_error_without_a_gpu():
    """Valid arguments on a host with no GPU: every entry point that needs the
    device returns HTTM_ERR_DEVICE with a message (never a crash), and the
    test hook's forced failure is reported as such."""
    w = gen.WORKLOADS["tiny"]
    plan = H.Plan.from_workload(w)
    L = H.lib()
    fake = [0x10000 * (i + 1) for i in range(5)]  # aligned, never dereferenced on the host
    st = L.httm_layer(plan.handle, fake[0], plan.workspace_bytes, fake[1], fake[2], fake[3], fake[4], None, None)
    assert st == 5 and L.httm_last_error().decode()
    assert L.httm_layer_noalloc(plan.handle, fake[1], fake[2], fake[3], fake[4], None) == 5
    assert L.httm_attention_dense(plan.handle, fake[0], plan.dense_workspace_bytes, fake[1], fake[2], fake[3], fake[4],
                                  None) == 5
    H.debug_fail_launch(1)
    st = L.httm_attention_dense(plan.handle, fake[0], plan.dense_workspace_bytes, fake[1], fake[2], fake[3], fake[4],
                                None)
    assert st == 5 and "forced launch failure" in L.httm_last_error().decode()
    H.debug_fail_launch(0)


def test_peak_mfma_validation():
    """The micro-benchmark entry point refuses a NULL output and iteration or
    grid counts out of range before anything is enqueued (no device needed)."""
    L = H.lib()
    fake = 0x10000
    flop = ctypes.c_double(-1.0)
    assert L.httm_peak_mfma(16, 4, 1.0, 1.0, None, None, ctypes.byref(flop)) == 1
    assert L.httm_peak_mfma(0, 4, 1.0, 1.0, fake, None, ctypes.byref(flop)) == 1
    assert L.httm_peak_mfma(12, 4, 1.0, 1.0, fake, None, ctypes.byref(flop)) == 1  # not a multiple of 8
    assert L.httm_peak_mfma((1 << 30) + 1, 4, 1.0, 1.0, fake, None, ctypes.byref(flop)) == 1
    assert L.httm_peak_mfma(16, 0, 1.0, 1.0, fake, None, ctypes.byref(flop)) == 1
    assert L.httm_peak_mfma(16, (1 << 20) + 1, 1.0, 1.0, fake, None, ctypes.byref(flop)) == 1
    assert flop.value == -1.0 and L.httm_last_error().decode()
    assert L.httm_peak_mfma_fp8(16, 4, None, None, ctypes.byref(flop)) == 1
    assert L.httm_peak_mfma_fp8(6, 4, fake, None, ctypes.byref(flop)) == 1  # not a multiple of 4
    assert L.httm_peak_mfma_fp8(16, 0, fake, None, ctypes.byref(flop)) == 1
    assert flop.value == -1.0


@pytest.mark.skipif(not _no_gpu(), reason="checks the error path of a host without a GPU")
def test_peak_mfma_without_a_gpu():
    """Valid arguments on a host with no GPU: the launch is reported as a
    device error, and the FLOP count follows from the arguments alone."""
    flop = ctypes.c_double(0.0)
    assert H.lib().httm_peak_mfma(24, 5, 1.0, 1.0, 0x10000, None, ctypes.byref(flop)) == 5
    assert flop.value == 24 * 5 * 4 * 8 * (2 * 16 * 16 * 32)


def test_index_import_refuses_bad_payloads():
    """An index assembled on the host: the size and the header are checked,
    then the payload (offsets rising from 0 to N, member ids below N, packed
    rows inside their head, lengths within the packed capacity) before any
    device copy; garbage behind a valid header is refused."""
    for name, kw in [("tiny", {}), ("tiny", {"partition": 1}), ("tiny", {"partition": 2}),
                     ("vggt30", {"heads": 2, "frames": 3})]:
        w = gen.WORKLOADS[name].with_(**kw)
        plan = H.Plan.from_workload(w)
        hdr = H.index_header(plan)
        assert hdr[:4].view(np.uint32)[0] == 0x58495448  # "HTIX"
        n = plan.index_bytes
        rng = np.random.default_rng(3)
        payloads = {"zeros": np.zeros(n, np.uint8),
                    "random": rng.integers(0, 256, n).astype(np.uint8),
                    "plausible": (np.arange(n // 4) % w.n_tokens).astype(np.int32).view(np.uint8)}
        L = H.lib()
        idx = H.Index(0, 0x10000, n, 0)  # never written: refused before any copy
        for what, buf in payloads.items():
            b = buf.copy()
            b[:64] = hdr
            st = L.httm_index_import(plan.handle, b.ctypes.data, n, ctypes.byref(idx), None)
            assert st == 4 and "out of range" in L.httm_last_error().decode(), (name, kw, what)
            assert idx.valid == 0
        b = payloads["zeros"].copy()
        assert L.httm_index_import(plan.handle, b.ctypes.data, n, ctypes.byref(idx), None) == 4  # no header
        b[:64] = hdr
        assert L.httm_index_import(plan.handle, b.ctypes.data, n - 4, ctypes.byref(idx), None) == 4  # size


ASAN_SKIP = "sanitized run in progress"


@pytest.mark.skipif(os.environ.get("HTTM_SANITIZED_RUN") == "1", reason=ASAN_SKIP)
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    """The host code (validation, plans, layouts, index checks, the error
    paths) built with AddressSanitizer and UndefinedBehaviorSanitizer, with
    the same kernel objects, and this module's tests run against it."""
    import shutil
    import subprocess
    import sys
    from token_merged_global_amd import build as B

    hipcc = B.hipcc()
    rt = sorted(__import__("glob").glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    kernels = [os.path.join(B.BUILD_DIR, f) for f in sorted(os.listdir(B.BUILD_DIR))
               if f.endswith(".hip.o")] if os.path.isdir(B.BUILD_DIR) else []
    if len(kernels) < 8:
        B.build()
        kernels = [os.path.join(B.BUILD_DIR, f) for f in sorted(os.listdir(B.BUILD_DIR)) if f.endswith(".hip.o")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    obj = str(tmp_path / "httm_asan.o")
    so = str(tmp_path / "libhttm.so")
    subprocess.run([hipcc, "-x", "hip", "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
                    "-I", os.path.join(ROOT, "include"), "-I", B.CSRC, *B.DEVICE_FLAGS, *san, "-c",
                    os.path.join(B.CSRC, "httm.cpp"), "-o", obj], check=True, capture_output=True, text=True)
    subprocess.run([hipcc, f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-shared-libsan", *san, "-o", so, obj,
                    *kernels], check=True, capture_output=True, text=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt[-1] + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HTTM_SANITIZED_RUN"] = "1"
    code = ("import sys, pytest; sys.path.insert(0, %r); import token_merged_global_amd as H; H.LIB_PATH = %r; "
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))") % (ROOT, so, os.path.abspath(__file__))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
