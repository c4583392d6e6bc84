"""Builds the gfx950 BA-Att shared library in-tree with hipcc.

    python -m block_sparse_attention_ba_amd.build

produces block_sparse_attention_ba_amd/libba_att.so from csrc/ba_att.hip
(one translation unit: host entry points plus the kernel headers) and
libba_peaks.so, the machine-peak microbenchmarks, from csrc/peaks.hip.
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
PEAKS_PATH = os.path.join(PKG, "libba_peaks.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the BA-Att library needs ROCm's hipcc to build")


def compile_command(out: str, source: str = "ba_att.hip") -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # inputs are finite: max/min need no NaN-quieting canonicalisation
        "-fno-honor-nans",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
        os.path.join(CSRC, source), "-o", out,
    ]


def _build_one(source: str, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = compile_command(tmp, source)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {source} ({res.returncode}):\n{res.stderr[-4000:]}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    _build_one("ba_att.hip", LIB_PATH, verbose)
    _build_one("peaks.hip", PEAKS_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
