"""Build libpa.so (the C ABI in include/pa.h and include/pa_manager.h) and
libpa_bench.so (the reference read kernels of include/pa_bench.h, used by
the benchmark only) with hipcc for gfx950.

Run as ``python -m paged_kv_cache_05_amd._build``; ``__graft_entry__.build()``
calls :func:`build`.  The library is built in-tree, next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["pa_api.hip", "pa_decode.hip", "pa_prefill.hip", "pa_cache.hip", "pa_plan.cpp",
           "pa_manager.cpp"]
LIBRARY = os.path.join(HERE, "libpa.so")
BENCH_SOURCES = ["pa_bench.hip"]
BENCH_LIBRARY = os.path.join(HERE, "libpa_bench.so")
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for all device code.  MFMA results
# stay in arch VGPRs (the prefill kernel's accumulators are rescaled by VALU
# code; in AGPRs every such use costs a move each way); kernels without MFMA
# compile to the same code either way.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def command(output: str, sources=None) -> list[str]:
    return ([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-I", os.path.join(ROOT, "include")] + DEVICE_FLAGS +
            ["-o", output] + [os.path.join(CSRC, s) for s in (sources or SOURCES)])


def _compile(library: str, sources, verbose: bool) -> str:
    tmp = library + ".tmp"
    cmd = command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature; drop that note.
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, library)
    return library


def build(verbose: bool = False) -> str:
    """Compile both libraries; returns the path of libpa.so."""
    _compile(BENCH_LIBRARY, BENCH_SOURCES, verbose)
    return _compile(LIBRARY, SOURCES, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
