"""Build libpa.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m paged_kv_attention_22_amd.build

Each source compiles to an object under _build/; the objects link into
paged_kv_attention_22_amd/libpa.so.  Always rebuilds (a build is a few tens of
seconds with parallel compiles).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "libpa")
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["kv_write.hip", "qkv_write.hip", "attn_rows.hip", "attn_chunks.hip", "pa_api.cpp",
           "noalloc.hip", "block_manager.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def common_flags() -> list[str]:
    return ["-O3", "-fPIC", "-std=c++17", "-Wall", f"--offload-arch={ARCH}",
            # no packed-fp32 instructions in device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in ordinary VGPRs: the softmax and rescaling
            # touch them with vector instructions, and AGPR accumulators then
            # cost a copy each way per tile
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(line for line in r.stderr.splitlines()
                    if "packed-fp32-ops" not in line)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
