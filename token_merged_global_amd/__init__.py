"""Python binding of the HTTM layer library (``include/httm.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libhttm.so``.  PyTorch provides device memory and the stream.  There is no
fallback: if the library is missing the import of ``lib()`` raises.

    plan = Plan(heads=16, d_head=64, frames=30, grid_h=37, grid_w=37,
                n_special=5, n_s=128, n_t=30, q_ratio=0.9, kv_ratio=0.5,
                outlier_pct=10.0, dtype="bf16")
    out = layer(plan, q, k, v)                       # q, k, v: [h][N][64] cuda tensors
    out, idx = layer(plan, q, k, v, keep_index=True)
    out2 = layer_cached(plan, idx, q2, k2, v2)       # reuse merge indices
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Dict, List, Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhttm.so")

HTTM_F32, HTTM_BF16 = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
          4: "index mismatch", 5: "device error"}
DEBUG_ITEMS = ["q_match", "q_score", "kv_match", "kv_score", "q_group", "kv_group", "delta",
               "outlier", "q_slot", "cu_q", "select", "attn_fallback",
               "ga_var", "ga_role", "ga_match", "ga_score", "kv_len", "kt", "vt", "qt",
               "gm_metric", "gm_match", "gm_score", "k8", "kexp", "q8", "qexp"]
#: Items that exist only with FP8 scores (attn_fp8).
FP8_ITEMS = ["k8", "kexp", "q8", "qexp"]
#: Items that exist only under one partition (block-local / geometry-aware / head-shared).
BLOCK_ITEMS = ["q_match", "q_score", "kv_match", "kv_score"]
GA_ITEMS = ["ga_var", "ga_role", "ga_match", "ga_score", "kv_len"]
GM_ITEMS = ["gm_metric", "gm_match", "gm_score"]
TIMING_STAGES = ["sim", "select", "merge_kv", "merge_q", "outlier", "restore", "attn", "unmerge", "attn_tail",
                 "ga_match", "sim_k", "select_k", "key_fp8"]


class HttmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"httm: {STATUS.get(status, status)}: {detail}")
        self.status = status


class Params(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("d_head", ctypes.c_int32), ("frames", ctypes.c_int32),
                ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("n_special", ctypes.c_int32),
                ("n_s", ctypes.c_int32), ("n_t", ctypes.c_int32), ("q_ratio", ctypes.c_double),
                ("kv_ratio", ctypes.c_double), ("outlier_pct", ctypes.c_double),
                ("q_dst_stride", ctypes.c_int32), ("kv_dst_stride", ctypes.c_int32),
                ("block_order", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("partition", ctypes.c_int32), ("protect_pct", ctypes.c_double),
                ("attn_split", ctypes.c_int32), ("attn_fp8", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("n_patch", ctypes.c_int64), ("n_blocks", ctypes.c_int32),
                ("q_stride", ctypes.c_int32), ("kv_stride", ctypes.c_int32), ("q_groups", ctypes.c_int64),
                ("kv_len", ctypes.c_int64), ("n_outliers", ctypes.c_int64), ("q_capacity", ctypes.c_int64),
                ("q_src", ctypes.c_int64), ("kv_src", ctypes.c_int64), ("softmax_scale", ctypes.c_float)]


BLOCK_FIELDS = ["start", "n", "f0", "nf", "j0", "run", "q_dst", "q_src", "q_r", "kv_dst", "kv_src",
                "kv_r", "q_slot0", "kv_slot0", "q_src0", "kv_src0"]


class Block(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in BLOCK_FIELDS]


class Index(ctypes.Structure):
    _fields_ = [("plan_id", ctypes.c_uint64), ("dev", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
                ("valid", ctypes.c_int32)]


EXPORTS = {
    "httm_plan_create": ([ctypes.POINTER(Params), ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
    "httm_plan_destroy": ([ctypes.c_void_p], None),
    "httm_plan_get_info": ([ctypes.c_void_p, ctypes.POINTER(PlanInfo)], ctypes.c_int),
    "httm_plan_get_blocks": ([ctypes.c_void_p, ctypes.POINTER(Block), ctypes.c_int32], ctypes.c_int),
    "httm_workspace_size": ([ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "httm_index_size": ([ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "httm_dense_workspace_size": ([ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "httm_layer": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                    ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Index), ctypes.c_void_p], ctypes.c_int),
    "httm_layer_cached": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Index),
                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                           ctypes.c_void_p], ctypes.c_int),
    "httm_index_export": ([ctypes.c_void_p, ctypes.POINTER(Index), ctypes.c_void_p, ctypes.c_size_t,
                           ctypes.c_void_p], ctypes.c_int),
    "httm_index_import": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(Index),
                           ctypes.c_void_p], ctypes.c_int),
    "httm_attention_dense": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p],
                             ctypes.c_int),
    "httm_debug_size": ([ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "httm_debug_read": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(Index), ctypes.c_int32, ctypes.c_void_p,
                         ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "httm_set_timing": ([ctypes.c_int32], ctypes.c_int),
    "httm_get_timing": ([ctypes.POINTER(ctypes.c_float), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)],
                        ctypes.c_int),
    "httm_noalloc_capacity": ([ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "httm_layer_noalloc": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.c_void_p], ctypes.c_int),
    "httm_index_header": ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t], ctypes.c_int),
    "httm_debug_fail_launch": ([ctypes.c_int32], ctypes.c_int),
    "httm_peak_mfma": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "httm_peak_mfma_fp8": ([ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                            ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "httm_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "httm_last_error": ([], ctypes.c_char_p),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded in-tree library; raises if it was not built (no fallback exists)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m token_merged_global_amd.build` (the HTTM layer has no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in EXPORTS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        raise HttmError(status, lib().httm_last_error().decode())


def _dtype_code(dtype) -> int:
    s = str(dtype)
    if s in ("bf16", "torch.bfloat16"):
        return HTTM_BF16
    if s in ("f32", "fp32", "torch.float32"):
        return HTTM_F32
    raise ValueError(f"unsupported dtype {dtype}")


class Plan:
    """Host-side plan: validated parameters, block table, buffer sizes."""

    def __init__(self, heads: int, frames: int, grid_h: int, grid_w: int, n_special: int, n_s: int,
                 n_t: int, q_ratio: float, kv_ratio: float, outlier_pct: float, dtype="bf16",
                 d_head: int = 64, q_dst_stride: int = 0, kv_dst_stride: int = 0, block_order: int = 0,
                 softmax_scale: float = 0.0, partition: int = 0, protect_pct: float = 10.0, attn_split: int = 0,
                 attn_fp8: bool = False):
        self.params = Params(heads, d_head, frames, grid_h, grid_w, n_special, n_s, n_t, float(q_ratio),
                             float(kv_ratio), float(outlier_pct), q_dst_stride, kv_dst_stride, block_order,
                             float(softmax_scale), _dtype_code(dtype), int(partition), float(protect_pct),
                             int(attn_split), int(bool(attn_fp8)))
        h = ctypes.c_void_p()
        _check(lib().httm_plan_create(ctypes.byref(self.params), ctypes.byref(h)))
        self.handle = h
        inf = PlanInfo()
        _check(lib().httm_plan_get_info(self.handle, ctypes.byref(inf)))
        self.info = {f: getattr(inf, f) for f, _ in PlanInfo._fields_}
        self.dtype = "bf16" if self.params.dtype == HTTM_BF16 else "f32"

    @staticmethod
    def from_workload(w, **kw) -> "Plan":
        args = dict(heads=w.heads, frames=w.frames, grid_h=w.grid_h, grid_w=w.grid_w, n_special=w.n_special,
                    n_s=w.n_s, n_t=w.n_t, q_ratio=w.q_ratio, kv_ratio=w.kv_ratio, outlier_pct=w.outlier_pct,
                    dtype=w.dtype, d_head=w.d_head, q_dst_stride=w.q_dst_stride,
                    kv_dst_stride=w.kv_dst_stride, softmax_scale=w.softmax_scale,
                    block_order=getattr(w, "block_order", 0), partition=getattr(w, "partition", 0),
                    protect_pct=getattr(w, "protect_pct", 10.0), attn_fp8=getattr(w, "attn_fp8", False))
        args.update(kw)
        return Plan(**args)

    def __del__(self):
        if getattr(self, "handle", None) and _LIB is not None:
            _LIB.httm_plan_destroy(self.handle)
            self.handle = None

    def _size(self, fn) -> int:
        n = ctypes.c_size_t()
        _check(fn(self.handle, ctypes.byref(n)))
        return n.value

    @property
    def workspace_bytes(self) -> int:
        return self._size(lib().httm_workspace_size)

    @property
    def index_bytes(self) -> int:
        return self._size(lib().httm_index_size)

    @property
    def dense_workspace_bytes(self) -> int:
        return self._size(lib().httm_dense_workspace_size)

    def blocks(self) -> List[Dict[str, int]]:
        n = self.info["n_blocks"]
        arr = (Block * n)()
        _check(lib().httm_plan_get_blocks(self.handle, arr, n))
        return [{f: getattr(b, f) for f in BLOCK_FIELDS} for b in arr]


# ----------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _stream_ptr(stream) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_qkv(plan: Plan, *ts) -> None:
    torch = _torch()
    want = torch.bfloat16 if plan.dtype == "bf16" else torch.float32
    shape = (plan.params.heads, plan.info["n_tokens"], plan.params.d_head)
    for t in ts:
        if not t.is_cuda or t.dtype != want or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"expected contiguous cuda {want} tensors of shape {shape}")


def workspace(plan: Plan, kind: str = "layer"):
    torch = _torch()
    n = plan.dense_workspace_bytes if kind == "dense" else plan.workspace_bytes
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def _on(stream):
    """Allocation context of the stream a call runs on.

    Buffers that a call allocates for itself (a temporary workspace, a fresh
    output) are taken from the caching allocator under the stream the
    kernels run on, so that the allocator orders their reuse after that
    stream's work (a block taken under another stream could be handed out
    again while this call's kernels still run)."""
    torch = _torch()
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


class CachedIndex:
    """Device buffer holding the merge indices of one layer (LiteVGGT-style reuse)."""

    def __init__(self, plan: Plan):
        torch = _torch()
        self.buf = torch.empty(plan.index_bytes, dtype=torch.uint8, device="cuda")
        self.c = Index(0, self.buf.data_ptr(), self.buf.numel(), 0)


def layer(plan: Plan, q, k, v, ws=None, out=None, index: Optional[CachedIndex] = None, stream=None,
          keep_index: bool = False):
    """One HTTM layer on the GPU.  Returns ``out`` (and the index if ``keep_index``)."""
    torch = _torch()
    _check_qkv(plan, q, k, v)
    with _on(stream):
        ws = workspace(plan) if ws is None else ws
        out = torch.empty_like(q) if out is None else out
        if keep_index and index is None:
            index = CachedIndex(plan)
    _check(lib().httm_layer(plan.handle, ws.data_ptr(), ws.numel(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            out.data_ptr(), ctypes.byref(index.c) if index is not None else None,
                            _stream_ptr(stream)))
    return (out, index) if keep_index else out


def layer_cached(plan: Plan, index: CachedIndex, q, k, v, ws=None, out=None, stream=None):
    """A layer reusing ``index`` from an earlier ``layer`` call with the same plan."""
    torch = _torch()
    _check_qkv(plan, q, k, v)
    with _on(stream):
        ws = workspace(plan) if ws is None else ws
        out = torch.empty_like(q) if out is None else out
    _check(lib().httm_layer_cached(plan.handle, ws.data_ptr(), ws.numel(), ctypes.byref(index.c),
                                   q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   _stream_ptr(stream)))
    return out


def noalloc_capacity() -> int:
    """Bytes of the library's static device scratch used by ``layer_noalloc``."""
    n = ctypes.c_size_t()
    _check(lib().httm_noalloc_capacity(ctypes.byref(n)))
    return n.value


def layer_noalloc(plan: Plan, q, k, v, out, stream=None):
    """One layer that allocates nothing: the library's static scratch is its
    workspace (plans up to ``noalloc_capacity()`` bytes of workspace); every
    launch goes to ``stream``.  ``out`` is the caller's output tensor."""
    _check_qkv(plan, q, k, v, out)
    _check(lib().httm_layer_noalloc(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    _stream_ptr(stream)))
    return out


def index_header(plan: Plan):
    """The 64-byte header (numpy uint8) that an index of ``plan`` starts with."""
    import numpy as np
    buf = np.zeros(64, dtype=np.uint8)
    _check(lib().httm_index_header(plan.handle, buf.ctypes.data, buf.nbytes))
    return buf


def debug_fail_launch(n: int) -> None:
    """Test hook: the n-th checked launch from now on reports a device error (0: off)."""
    _check(lib().httm_debug_fail_launch(int(n)))


PEAK_THREADS = 256  # lanes per workgroup of httm_peak_mfma


def peak_mfma(iters: int, grid: int, out, a: float = 1.0, b: float = 1.0, stream=None) -> float:
    """Enqueue the MFMA peak micro-benchmark (httm_peak_mfma) into ``out``
    (contiguous cuda float32, at least grid * PEAK_THREADS elements); returns
    the launch's MFMA FLOP."""
    torch = _torch()
    if not out.is_cuda or out.dtype != torch.float32 or not out.is_contiguous() or \
            out.numel() < int(grid) * PEAK_THREADS:
        raise ValueError(f"out must be a contiguous cuda float32 tensor of at least {int(grid) * PEAK_THREADS} elements")
    flop = ctypes.c_double(0.0)
    _check(lib().httm_peak_mfma(int(iters), int(grid), float(a), float(b), out.data_ptr(), _stream_ptr(stream),
                                ctypes.byref(flop)))
    return flop.value


def peak_mfma_fp8(iters: int, grid: int, out, stream=None) -> float:
    """Enqueue the FP8 MFMA peak micro-benchmark (httm_peak_mfma_fp8); returns the launch's FLOP."""
    torch = _torch()
    if not out.is_cuda or out.dtype != torch.float32 or not out.is_contiguous() or \
            out.numel() < int(grid) * PEAK_THREADS:
        raise ValueError(f"out must be a contiguous cuda float32 tensor of at least {int(grid) * PEAK_THREADS} elements")
    flop = ctypes.c_double(0.0)
    _check(lib().httm_peak_mfma_fp8(int(iters), int(grid), out.data_ptr(), _stream_ptr(stream), ctypes.byref(flop)))
    return flop.value


def index_export(plan: Plan, index: CachedIndex, stream=None):
    """Host copy (numpy uint8) of an index filled by ``layer`` with this plan."""
    import numpy as np
    buf = np.empty(plan.index_bytes, dtype=np.uint8)
    _check(lib().httm_index_export(plan.handle, ctypes.byref(index.c), buf.ctypes.data, buf.nbytes,
                                   _stream_ptr(stream)))
    return buf


def index_import(plan: Plan, host, stream=None) -> CachedIndex:
    """A device index holding ``host`` (bytes exported with a plan of the same parameters)."""
    import numpy as np
    buf = np.ascontiguousarray(np.frombuffer(memoryview(host), dtype=np.uint8))
    index = CachedIndex(plan)
    _check(lib().httm_index_import(plan.handle, buf.ctypes.data, buf.nbytes, ctypes.byref(index.c),
                                   _stream_ptr(stream)))
    return index


def attention_dense(plan: Plan, q, k, v, ws=None, out=None, stream=None):
    """Unmerged softmax(scale q k^T) v per head on the same attention kernel."""
    torch = _torch()
    _check_qkv(plan, q, k, v)
    with _on(stream):
        ws = workspace(plan, "dense") if ws is None else ws
        out = torch.empty_like(q) if out is None else out
    _check(lib().httm_attention_dense(plan.handle, ws.data_ptr(), ws.numel(), q.data_ptr(), k.data_ptr(),
                                      v.data_ptr(), out.data_ptr(), _stream_ptr(stream)))
    return out


#: Merged rows (K~, V~^T, Q~): as large as the inputs, read only on request.
ROW_ITEMS = ["kt", "vt", "qt"]


def debug_items(plan: Plan, rows: bool = False) -> List[str]:
    """The debug items that exist for ``plan``'s partition (merged rows only if ``rows``)."""
    part = plan.params.partition
    keep = {0: BLOCK_ITEMS, 1: GA_ITEMS, 2: GM_ITEMS}[part]
    skip = [it for it in BLOCK_ITEMS + GA_ITEMS + GM_ITEMS if it not in keep]
    if not plan.params.attn_fp8:
        skip += FP8_ITEMS
    return [it for it in DEBUG_ITEMS if it not in skip and (rows or it not in ROW_ITEMS + FP8_ITEMS)]


def debug_read(plan: Plan, ws, item: str, stream=None, index: Optional[CachedIndex] = None):
    """Copy one intermediate of the last ``layer`` on ``ws`` to a numpy array.

    Pass the ``index`` that call filled, if any (per-token slots live there).
    """
    import numpy as np
    code = DEBUG_ITEMS.index(item)
    n = ctypes.c_size_t()
    _check(lib().httm_debug_size(plan.handle, code, ctypes.byref(n)))
    rows = np.uint16 if plan.dtype == "bf16" else np.float32  # merged rows: bf16 bit patterns or fp32
    dt = {"q_score": np.float32, "kv_score": np.float32, "delta": np.float32, "outlier": np.uint8,
          "select": np.uint32, "ga_var": np.float32, "ga_role": np.uint8,
          "ga_score": np.float32, "kt": rows, "vt": rows, "qt": rows, "gm_metric": rows,
          "gm_score": np.float32, "k8": np.uint8, "q8": np.uint8}.get(item, np.int32)
    arr = np.empty(n.value // np.dtype(dt).itemsize, dtype=dt)
    _check(lib().httm_debug_read(plan.handle, ws.data_ptr(), ctypes.byref(index.c) if index is not None else None,
                                 code, arr.ctypes.data, arr.nbytes, _stream_ptr(stream)))
    return arr


TIMING_SERIAL = 1 << 30


def set_timing(stages=None, serial: bool = False) -> None:
    """Record HIP events around the named stages of the next calls (None: all, []: off).

    ``serial``: while timing, layers run every launch on the caller's stream
    (no concurrent key branch), so each stage times its kernels alone."""
    names = TIMING_STAGES if stages is None else list(stages)
    mask = 0
    for n in names:
        mask |= 1 << TIMING_STAGES.index(n)
    if serial and mask:
        mask |= TIMING_SERIAL
    _check(lib().httm_set_timing(mask))


def get_timing() -> Tuple[Dict[str, float], int]:
    """(mean ms per stage over the recorded calls, number of recorded calls)."""
    arr = (ctypes.c_float * len(TIMING_STAGES))()
    calls = ctypes.c_int32()
    _check(lib().httm_get_timing(arr, len(TIMING_STAGES), ctypes.byref(calls)))
    return {s: float(arr[i]) for i, s in enumerate(TIMING_STAGES)}, calls.value
