"""Build the HIP library ``libgemm_bf16.so`` in-tree with hipcc for gfx950.

Usage: ``python -m bf16_gemm_fp32_amd.build``.  Cross-compiles without a GPU.
Each translation unit (host launcher, one per tile configuration) compiles in
its own process; the objects are then linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libgemm_bf16.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SOURCES = ["gemm_bf16.hip", "tile_large.hip", "tile_medium.hip", "tile_medium_masked.hip", "tile_ring.hip", "tile_ring_w8.hip", "tile_ring_masked.hip", "tile_ring_q8.hip", "tile_ring_q8_exact.hip", "tile_fp8.hip", "tile_fp8_masked.hip", "tile_fp8_medium.hip", "tile_fp8_ring16.hip", "tile_ring_mfma32.hip", "tile_skinny.hip", "tile_skinny_t.hip", "tile_skinny_fp8.hip", "tile_skinny_q8.hip", "tile_gemv.hip"]

# Packed-fp32 VALU forms are disabled: the kernels write plain float code.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_files() -> list:
    """Every file the library is compiled from (kernels, launchers, C header)."""
    files = glob.glob(os.path.join(CSRC, "*.h")) + glob.glob(os.path.join(CSRC, "*.hip"))
    files += glob.glob(os.path.join(INCLUDE, "*.h"))
    return sorted(files)


def source_digest() -> str:
    """Short SHA-256 over the library sources (path and bytes of each file).
    Hardware-counter results recorded for one digest describe exactly that
    code; any edit to a kernel, a launcher or the header changes it."""
    h = hashlib.sha256()
    for path in source_files():
        h.update(os.path.relpath(path, ROOT).encode())
        h.update(b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="gemm_bf16_build_") as tmp:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([HIPCC, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        out = LIB_PATH + ".tmp"
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out, *objs], verbose)
        os.replace(out, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    if "--digest" in sys.argv:
        print(source_digest())
    else:
        print(build(verbose="-q" not in sys.argv))
