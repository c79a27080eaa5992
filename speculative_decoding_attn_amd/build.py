"""Compile the HIP sources into the in-tree shared library ``libeagle_mi355.so``.

    python -m speculative_decoding_attn_amd.build

gfx950 only; every HIP translation unit is built with packed-fp32 instructions
disabled.  Objects go to ``_build/`` at the repository root.
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
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libeagle_mi355.so")
SOURCES = ["api.hip", "tree_attn.hip", "lm_head.hip", "accept.hip", "rerank.hip", "kv_commit.hip",
           "draft.hip", "calib.hip"]
ARCH = "gfx950"
# Per-source options.  Tree attention: MFMA results in VGPRs (the four-wave kernel's
# vector work reads its scores and rescales its output in place; with accumulators in
# AGPRs the register allocator spills the loop state).
EXTRA = {"tree_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
        cmd = [hipcc, *flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if verbose or r.returncode:
            out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                            if "packed-fp32-ops" not in l)
            if out.strip():
                print(out, file=sys.stderr)
        if r.returncode:
            raise RuntimeError(f"hipcc failed on {src}")
        return obj

    with ThreadPoolExecutor(min(jobs, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        print(r.stdout + r.stderr, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
