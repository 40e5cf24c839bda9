"""Builds libmcs.so, the HIP library behind include/mcs.h, for gfx950.

    python -m token_sparse_attention_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The library lands next to
this file so that it travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmcs.so")
ARCH = os.environ.get("MCS_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # never emit packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
]


# Per-source extra flags.  pddp.hip: MFMA accumulators in VGPRs (the
# direction kernel copies the node's moments into VGPRs for its VALU
# matrix-vector products anyway; with AGPR accumulators the unused copies
# count against occupancy).
EXTRA_FLAGS = {"pddp.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmcs)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links libmcs.so."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    objs = [os.path.join(objdir, os.path.basename(src) + ".o") for src in sources]
    cmds = [[hipcc(), *compile_flags, *EXTRA_FLAGS.get(os.path.basename(src), []),
             "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            for src, obj in zip(sources, objs)]
    with ThreadPoolExecutor(max(1, min(len(cmds), os.cpu_count() or 1, 8))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), *FLAGS, *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
