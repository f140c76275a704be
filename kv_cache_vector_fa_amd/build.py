"""Build the gfx950 shared library ``libfa_tq.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled and fp32 denormals kept (the encoder's fp32 results are defined bit for
bit, including tiny inputs).  The codec translation unit is compiled without
floating-point contraction, so a*b + c is never fused there.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfa_tq.so")
BUILD_DIR = os.path.join(ROOT, "_build")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]

SOURCES = [
    ("fa_tq_host.cpp", ["-x", "hip"]),
    ("codec.hip", ["-ffp-contract=off"]),
    ("attn.hip", []),
    ("attn_mfma.hip", []),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile all sources and link ``libfa_tq.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src, flags in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [hipcc()] + COMMON + flags + (extra or []) + ["-c", os.path.join(CSRC, src),
                                                            "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
