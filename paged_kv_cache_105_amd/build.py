"""Build the HIP library in-tree: paged_kv_cache_105_amd/libpkv.so (gfx950).

Run as ``python -m paged_kv_cache_105_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  hipcc cross-compiles for gfx950 without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpkv.so")
BENCH_LIB = os.path.join(PKG, "libpkv_bench.so")   # measurement helper of bench.py

HIP_SOURCES = ["kv_append.hip", "copy_blocks.hip", "decode_generic.hip", "decode_mfma.hip",
               "combine.hip", "chunk_attention.hip", "swap.hip", "noalloc.hip"]
CXX_SOURCES = ["api.cpp", "pool.cpp", "sha256.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile libpkv.so and the bench helper libpkv_bench.so (always recompiles)."""
    _compile([os.path.join(CSRC, s) for s in HIP_SOURCES + CXX_SOURCES], LIB, verbose)
    _compile([os.path.join(CSRC, "bench_gather.hip")], BENCH_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
