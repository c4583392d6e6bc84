"""Builds the gfx950 BA-Att shared library in-tree with hipcc.

    python -m block_sparse_attention_ba_amd.build

produces block_sparse_attention_ba_amd/libba_att.so from csrc/ba_att.hip
(one translation unit: host entry points plus the kernel headers).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libba_att.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the BA-Att library needs ROCm's hipcc to build")


def compile_command(out: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # inputs are finite: max/min need no NaN-quieting canonicalisation
        "-fno-honor-nans",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        os.path.join(CSRC, "ba_att.hip"), "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = compile_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
