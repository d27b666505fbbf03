"""Build libspecverify.so in-tree with hipcc for gfx950.

Usage: ``python -m draft_token_verification_chain_amd.build`` (or call
``build()``).  The shared library lands next to this file, where the Python
binding loads it from.
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libspecverify.so")
SOURCES = [os.path.join(CSRC, "specverify.hip")]
HEADERS = sorted(glob.glob(os.path.join(CSRC, "*.hpp"))) + [os.path.join(INCLUDE, "specverify.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no floating-point contraction except the fmas written out explicitly:
    # every kernel then evaluates a shared formula bit-identically
    "-ffp-contract=off",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wextra",
]


def build(verbose: bool = True) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
