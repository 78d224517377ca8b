"""Builds libfa.so, the gfx950 attention library, in place with hipcc.

Usage: python -m exact_io_aware_72_amd.build [-v]

Each source is compiled in its own hipcc process (in parallel), then linked
into one shared library next to this file. Cross-compiles on a machine
without a GPU.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB_PATH = os.path.join(HERE, "libfa.so")
POISON_LIB_PATH = os.path.join(HERE, "libfa_poison.so")  # race-detection build, tests only
CLOCK_LIB_PATH = os.path.join(HERE, "libfa_clock.so")    # benchmark clock stamps, not attention
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_noalloc.hip"]
CLOCK_SOURCES = ["clock_stamp.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # Packed fp32 VALU instructions stay off (the compiler would otherwise
    # form them from scalar or float2 code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results go to ordinary VGPRs, so the softmax and the
    # rescale read them without accumulator-register copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # No NaN quieting before max: lets row maxima use v_max3 on raw scores.
    "-fno-honor-nans",
    "-Wall",
    "-Wno-unused-function",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line and "is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)
    return out


def _build_lib(out_path: str, flags, verbose: bool, sources=None) -> None:
    cc = hipcc()
    sources = SOURCES if sources is None else sources
    tmp = tempfile.mkdtemp(prefix="fa_build_")
    try:
        objs = []
        jobs = []
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(sources)) as ex:
            for src in sources:
                obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
                objs.append(obj)
                cmd = [cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
                jobs.append(ex.submit(_run, cmd, verbose))
            for j in jobs:
                j.result()
        out_tmp = out_path + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs, verbose)
        os.replace(out_tmp, out_path)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compiles every source and links libfa.so, the race-detection build
    libfa_poison.so (the same sources with -DFA_LDS_POISON: LDS stages are
    filled with NaN bytes between their last read and the next tile's
    loads) and the benchmark's clock-stamp library libfa_clock.so; returns
    the path of libfa.so."""
    flags = COMMON_FLAGS + list(extra_flags or [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=3) as ex:
        jobs = [ex.submit(_build_lib, LIB_PATH, flags, verbose),
                ex.submit(_build_lib, POISON_LIB_PATH, flags + ["-DFA_LDS_POISON"], verbose),
                ex.submit(_build_lib, CLOCK_LIB_PATH, flags, verbose, CLOCK_SOURCES)]
        for j in jobs:
            j.result()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
