"""Builds the gfx950 HIP library ``libvdx_attn.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 VALU forms
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libvdx_attn.so")
SOURCES = [os.path.join(CSRC, "attn_fwd_kernel.hip"), os.path.join(CSRC, "natten_fwd_kernel.hip"),
           os.path.join(CSRC, "attn_bwd_kernel.hip"), os.path.join(CSRC, "rope3d_kernel.hip"),
           os.path.join(CSRC, "vdx_attn_api.hip")]

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-fvisibility=hidden", "-Wall", "-fno-honor-nans",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build_library(verbose: bool = False, out: str = LIB_PATH, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
