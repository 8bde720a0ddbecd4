"""Builds the CPU oracle library (plain C, gcc, no fast-math, no FP contraction).

Test infrastructure: the library is loaded only by the tests, the smoke check
and the benchmark's CPU-baseline leg.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
NATTEN_SRC = os.path.join(HERE, "natten_oracle.c")
BWD_SRC = os.path.join(HERE, "attn_bwd_oracle.c")
ROPE_SRC = os.path.join(HERE, "rope_oracle.c")
LIB_PATH = os.path.join(HERE, "libvdx_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-pthread", "-Wall", "-Wextra", "-fvisibility=hidden"]


def build_oracle(verbose: bool = False, src: str = SRC, out: str = LIB_PATH,
                 natten_src: str = NATTEN_SRC, bwd_src: str = BWD_SRC, rope_src: str = ROPE_SRC) -> str:
    """One shared library from the oracle sources; ``src`` / ``natten_src`` /
    ``bwd_src`` / ``rope_src`` let the mutation tests swap in a modified copy
    of one."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, src, natten_src, bwd_src, rope_src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle(verbose=True))
