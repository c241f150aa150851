"""Compile the gfx950 HIP sources of the package into ``liboq.so`` (in-tree).

The library is built with hipcc for gfx950 only.  Packed float32 VALU
instructions are disabled on purpose (``-packed-fp32-ops``): every float32
operation in the kernels is a scalar-per-lane IEEE operation.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liboq.so")
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into liboq.so; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include")] + sources() + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (proc.stdout + proc.stderr).splitlines()
            if "packed-fp32-ops" not in ln and "recognized feature" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
