"""Build libpagedkv.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

    python -m paged_kv_cache_133_amd.build

Objects go to _build/ at the repository root; the library lands next to this file.
Every HIP file is compiled with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["api.hip", "write.hip", "norm_rope.hip", "decode.hip", "int8_kv.hip", "mla_wide.hip",
           "varlen_attn.hip", "gqa_attn.hip", "block_manager.hip",
           "runner.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]
# The MFMA attention kernels keep their accumulators in ordinary VGPRs: with the default
# choice (AGPRs) the online-softmax rescale copies every accumulator out and back each tile.
EXTRA = {"varlen_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "mla_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "gqa_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpagedkv.so")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
