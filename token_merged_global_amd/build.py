"""Compile the HIP/C++ sources of the HTTM layer library for gfx950.

``python -m token_merged_global_amd.build`` (or ``build()``) writes
``token_merged_global_amd/libhttm.so`` in-tree.  Sources compile in parallel
to objects under ``token_merged_global_amd/_build/`` and link into one shared
library with a plain C ABI (``include/httm.h``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libhttm.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

# Packed fp32 VALU ops are disabled for all device code (see DESIGN notes on
# the target); -O3 otherwise.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Sources whose arithmetic must be exactly the written sequence of rounded
# operations (means and deviations compared bit for bit): no FMA contraction.
PER_FILE = {"k_merge.hip": ["-ffp-contract=off"],
            # MFMA results in VGPRs: the softmax reads them with plain VALU ops
            "k_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            "k_attn8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            "k_sim.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            # without it the accumulators live in AGPRs and the loop copies them every iteration
            "k_peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            # variance map compared bit for bit; MFMA cosine tiles as in k_sim
            "k_ga.hip": ["-ffp-contract=off", "-mllvm", "-amdgpu-mfma-vgpr-form=1"],
            # head-shared metric: fp32 adds in head order and one division
            "k_global.hip": ["-ffp-contract=off"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-I", CSRC, "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HTTM library needs the ROCm toolchain to build")


def sources(csrc: str = CSRC):
    return sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".cpp")))


def _compile(src: str, verbose: bool, build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    extra = PER_FILE.get(os.path.basename(src), [])
    inc = ["-I", os.path.dirname(src)]
    cmd = [hipcc(), *lang, *COMMON, *inc, *DEVICE_FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int = 8, csrc: str = CSRC, out: str = OUT) -> str:
    """Compile every source of `csrc` for gfx950 and link `out` (default: the in-tree library)."""
    build_dir = BUILD_DIR if out == OUT else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources(csrc)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
