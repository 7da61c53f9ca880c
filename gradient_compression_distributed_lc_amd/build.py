"""Builds libtlc.so (the HIP library behind include/tlc.h) in-tree for gfx950.

    python -m gradient_compression_distributed_lc_amd.build

Flags: no fast-math, IEEE fp32 denormals kept, no floating-point
contraction, and packed-fp32 instructions disabled (the compiler otherwise
forms v_pk_* fp32 ops on its own).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "tlc.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libtlc.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off",
    "-Wall", "-Werror=return-type",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def command(out: str = LIB) -> list[str]:
    return [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, SRC, "-o", out]


def build(out: str = LIB, quiet: bool = True) -> str:
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    r = subprocess.run(command(tmp), capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {out}")
    if not quiet:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(quiet=False))
