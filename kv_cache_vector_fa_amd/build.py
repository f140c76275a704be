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
    ("dense.hip", ["-ffp-contract=off"]),
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


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libfa_tq_asan.so")
# AddressSanitizer on the host code only (-Xarch_host before each sanitizer flag):
# the device code is compiled as usual
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of hipcc's clang (to LD_PRELOAD into a
    process that loads the ASan build)."""
    out = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out


def build_asan(verbose: bool = False) -> str:
    """The host library fa_tq_host.cpp (argument checks, codebooks, signs, dispatch)
    compiled with AddressSanitizer and linked with the kernel objects of ``build``
    into ``_build/asan/libfa_tq_asan.so``; runs without a GPU for the host-side tests.
    Load it with the runtime from ``asan_runtime()`` preloaded."""
    objs = [os.path.join(BUILD_DIR, src + ".o") for src, _ in SOURCES[1:]]
    if not all(os.path.exists(o) for o in objs):
        build(verbose)
    os.makedirs(ASAN_DIR, exist_ok=True)
    host = os.path.join(ASAN_DIR, "fa_tq_host.o")
    src, flags = SOURCES[0]
    cmd = [hipcc()] + COMMON + flags + ASAN_HOST + ["-c", os.path.join(CSRC, src), "-o", host]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libasan"] + \
        ASAN_HOST + ["-o", ASAN_LIB, host] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
