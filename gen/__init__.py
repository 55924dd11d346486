"""Seeded synthetic Q/K/V for the HTTM global-attention layer.

This module only draws inputs. It holds none of the layer's arithmetic and is
the one piece of code that both the oracle side (tests, CPU baseline) and the
HIP side (tests, bench) use, so that both consume identical bytes.

The pages measure on 7Scenes, NRGBD, ETH3D, ScanNet-50, DTU and Tanks & Temples
with trained VGGT weights ("HTTM: Head-wise Temporal Token Merging for Faster
VGGT", experiments; "LiteVGGT", experiments). None of these is available, so
tokens are synthetic but shaped like VGGT's global-attention inputs: a 37x37
patch grid plus 5 special tokens per frame, 16 heads of 64 channels, and the
spatial-local plus temporal-correspondence redundancy that the HTTM page names
as the reason merging works (HTTM page, "research background", insight).

Value recipe, per (tensor in {q,k,v}, head), independent streams:

* patch token (f, y, x) = B[y, x] + D[f] + e[f, y, x] where
  B ~ N(0, 1)^d per grid cell smoothed by a 3x3 box filter (mean over the
  in-bounds neighbours), D[f] ~ N(0, 0.1^2)^d one drift per frame,
  e ~ N(0, 0.05^2)^d i.i.d. noise;
* special tokens (the first ``n_special`` slots of each frame) ~ N(0, 1)^d;
* layer l >= 1 of a cached stack: X_l = X_{l-1} + N(0, 0.02^2) on an fp32
  master copy.

Stream keys are ``SeedSequence([seed, cfg, layer, tensor, head])`` with draw
order base (H*W*d), drift (F*d), specials (F*n_sp*d), noise (F*H*W*d), so any
head can be regenerated on its own.  bf16 tensors are the round-to-nearest-even
bf16 rounding of the fp32 master.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
from dataclasses import dataclass, field, replace
from typing import Dict, Iterable, Iterator, List, Optional, Sequence, Tuple

import numpy as np

DEFAULT_SEED = 0x4854544D
TENSORS = ("q", "k", "v")


@dataclass(frozen=True)
class Workload:
    """Shape and parameters of one layer workload (no arithmetic here)."""

    name: str
    cfg_id: int
    dtype: str  # "f32" or "bf16"
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
    softmax_scale: float = 0.125
    q_dst_stride: int = 0
    kv_dst_stride: int = 0
    block_order: int = 0  # 0 frame-major, 1 frame-minor stacking inside a block
    partition: int = 0  # 0 HTTM temporal blocks, 1 geometry-aware three-class partition
    protect_pct: float = 10.0  # partition 1: percent of each frame's patches protected
    attn_fp8: bool = False  # attention scores from FP8 (e4m3) queries and keys
    layers: int = 1
    sigma_drift: float = 0.1
    sigma_noise: float = 0.05
    sigma_layer: float = 0.02

    @property
    def tokens_per_frame(self) -> int:
        return self.n_special + self.grid_h * self.grid_w

    @property
    def n_tokens(self) -> int:
        return self.frames * self.tokens_per_frame

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _vggt(name, cfg_id, frames, **kw) -> Workload:
    base = dict(dtype="bf16", heads=16, d_head=64, frames=frames, grid_h=37, grid_w=37,
                n_special=5, n_s=128, n_t=30, q_ratio=0.9, kv_ratio=0.5, outlier_pct=10.0)
    base.update(kw)
    return Workload(name=name, cfg_id=cfg_id, **base)


#: The five workloads: a tiny fp32 layer and VGGT-shaped layers at 30, 100,
#: 200 and 500 frames (37x37 patches + 5 specials, 16 heads x 64).
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload(name="tiny", cfg_id=0, dtype="f32", heads=1, d_head=64, frames=4,
                     grid_h=16, grid_w=16, n_special=0, n_s=64, n_t=4, q_ratio=0.5,
                     kv_ratio=0.5, outlier_pct=10.0),
    "vggt30": _vggt("vggt30", 1, 30),
    "vggt100": _vggt("vggt100", 2, 100),
    "vggt200": _vggt("vggt200", 3, 200),
    "vggt500": _vggt("vggt500", 4, 500, layers=6),
}


def _stream(seed: int, cfg_id: int, layer: int, tensor: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, layer, tensor, head])))


def _box3(a: np.ndarray) -> np.ndarray:
    """3x3 box filter over the first two axes, mean over in-bounds cells."""
    H, W = a.shape[:2]
    pad = np.zeros((H + 2, W + 2) + a.shape[2:], dtype=np.float64)
    cnt = np.zeros((H + 2, W + 2), dtype=np.float64)
    pad[1:-1, 1:-1] = a
    cnt[1:-1, 1:-1] = 1.0
    acc = np.zeros(a.shape, dtype=np.float64)
    c = np.zeros((H, W), dtype=np.float64)
    for dy in range(3):
        for dx in range(3):
            acc += pad[dy:dy + H, dx:dx + W]
            c += cnt[dy:dy + H, dx:dx + W]
    return (acc / c.reshape(H, W, *([1] * (a.ndim - 2)))).astype(np.float32)


def head_tensor(w: Workload, tensor: str, head: int, seed: int = DEFAULT_SEED,
                layer: int = 0, frames: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp32 master values [N][d] of one head of one tensor at ``layer``.

    ``frames`` is unused by the recipe and reserved; every call draws the
    whole head so that streams stay aligned.
    """
    ti = TENSORS.index(tensor)
    H, W, F, d, sp = w.grid_h, w.grid_w, w.frames, w.d_head, w.n_special
    rng = _stream(seed, w.cfg_id, 0, ti, head)
    base = _box3(rng.standard_normal((H, W, d), dtype=np.float32))
    drift = rng.standard_normal((F, d), dtype=np.float32) * np.float32(w.sigma_drift)
    spec = rng.standard_normal((F, sp, d), dtype=np.float32)
    noise = rng.standard_normal((F, H * W, d), dtype=np.float32) * np.float32(w.sigma_noise)
    x = np.empty((F, sp + H * W, d), dtype=np.float32)
    x[:, :sp] = spec
    x[:, sp:] = base.reshape(1, H * W, d) + drift[:, None, :] + noise
    x = x.reshape(F * (sp + H * W), d)
    for l in range(1, layer + 1):
        r = _stream(seed, w.cfg_id, l, ti, head)
        x += r.standard_normal(x.shape, dtype=np.float32) * np.float32(w.sigma_layer)
    return x


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of values that are already bf16-representable."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_inputs(w: Workload, seed: int = DEFAULT_SEED, layer: int = 0,
                 heads: Optional[Iterable[int]] = None, workers: int = 0) -> Dict[str, np.ndarray]:
    """q, k, v as fp32 arrays [len(heads)][N][d] holding the values both sides consume.

    For bf16 workloads the values are bf16-representable (already rounded).
    Heads are drawn in parallel threads (each head has its own stream).
    """
    hs = list(range(w.heads)) if heads is None else list(heads)
    out = {t: np.empty((len(hs), w.n_tokens, w.d_head), dtype=np.float32) for t in TENSORS}

    def one(job):
        t, i, h = job
        x = head_tensor(w, t, h, seed=seed, layer=layer)
        out[t][i] = round_bf16(x) if w.dtype == "bf16" else x

    jobs = [(t, i, h) for t in TENSORS for i, h in enumerate(hs)]
    with cf.ThreadPoolExecutor(max_workers=workers or default_workers()) as ex:
        list(ex.map(one, jobs))
    return out


def layer_stack(w: Workload, seed: int = DEFAULT_SEED, heads: Optional[Iterable[int]] = None,
                layers: Optional[int] = None, workers: int = 0) -> Iterator[Tuple[int, Dict[str, np.ndarray]]]:
    """Successive layers (layer, inputs) of a stack: layer l adds N(0, 0.02^2) to l-1.

    Keeps the fp32 masters of the listed heads and adds one noise draw per
    layer, so layer l costs one draw instead of l (same values as
    ``layer_inputs(w, seed, layer=l)``).
    """
    hs = list(range(w.heads)) if heads is None else list(heads)
    n_layers = w.layers if layers is None else layers
    master = {t: np.empty((len(hs), w.n_tokens, w.d_head), dtype=np.float32) for t in TENSORS}
    pool = cf.ThreadPoolExecutor(max_workers=workers or default_workers())
    try:
        def base(job):
            t, i, h = job
            master[t][i] = head_tensor(w, t, h, seed=seed, layer=0)

        jobs = [(t, i, h) for t in TENSORS for i, h in enumerate(hs)]
        list(pool.map(base, jobs))
        for l in range(n_layers):
            if l > 0:
                def step(job, l=l):
                    t, i, h = job
                    r = _stream(seed, w.cfg_id, l, TENSORS.index(t), h)
                    master[t][i] += r.standard_normal(master[t][i].shape, dtype=np.float32) * np.float32(w.sigma_layer)

                list(pool.map(step, jobs))
            yield l, {t: (round_bf16(master[t]) if w.dtype == "bf16" else master[t].copy()) for t in TENSORS}
    finally:
        pool.shutdown()


def oracle_heads(w: Workload, seed: int = DEFAULT_SEED, n: int = 2) -> List[int]:
    """The seeded head subset on which expensive oracle stages run."""
    return sorted(int(h) for h in np.random.default_rng(seed).choice(w.heads, n, replace=False))
