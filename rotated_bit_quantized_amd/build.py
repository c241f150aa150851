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
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _filter(text):
    return [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln and "recognized feature" not in ln]


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source (one hipcc process per file, in parallel) and
    link them into liboq.so; returns the library path."""
    import concurrent.futures
    import tempfile
    jobs = jobs or min(8, os.cpu_count() or 1)
    with tempfile.TemporaryDirectory(prefix="oq_build_") as tmpd:
        def compile_one(src):
            obj = os.path.join(tmpd, os.path.basename(src) + ".o")
            cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            proc = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, proc.returncode, _filter(proc.stdout + proc.stderr)

        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(compile_one, sources()))
        errors = [f"{os.path.basename(src)}:\n" + "\n".join(msgs) for src, _, rc, msgs in results if rc != 0]
        if errors:
            raise RuntimeError("hipcc failed:\n" + "\n".join(errors))
        if verbose:
            for src, _, _, msgs in results:
                if msgs:
                    print("\n".join(msgs), file=sys.stderr)
        tmp = LIB + ".tmp"
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + [obj for _, obj, _, _ in results] + ["-o", tmp]
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError("link failed:\n" + "\n".join(_filter(proc.stdout + proc.stderr)))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
