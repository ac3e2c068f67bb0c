"""Build libptb.so for gfx950 with hipcc, in-tree.

    python -m transformer_block_amd.build

Each source is compiled to an object under ``transformer_block_amd/_build``
(in parallel), then linked into ``transformer_block_amd/libptb.so``.  Every
call rebuilds from source.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libptb.so")
SOURCES = ["gemm.hip", "attention_fwd.hip", "attention.hip", "layernorm.hip", "lamb.hip", "fp8_cast.hip",
           "dropout.hip",
           "ptb_api.cpp"]
# Per-source code generation options.  The attention forward rescales its
# output accumulators with vector ALU instructions; with the accumulators in
# AGPRs the compiler copies all of them to VGPRs on every key tile, so there
# the matrix-core results go to VGPRs.  (The backward kernels, which hold
# twice the accumulators, are faster with the default.)
EXTRA_FLAGS = {"attention_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libptb)")


def common_flags() -> list:
    return [
        "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
        # keep hipcc from emitting packed fp32 arithmetic (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
