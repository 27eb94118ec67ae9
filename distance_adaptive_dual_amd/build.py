"""Compile the DAR HIP library (``libdar.so``) and the benchmark's calibration
library (``libdar_calib.so``) for gfx950 with hipcc.

The library is built in-tree, next to this file, so it travels with the
source tree.  ``python -m distance_adaptive_dual_amd.build`` rebuilds it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdar.so")
SOURCES = ["dar_api.cpp", "rope.hip", "gemm.hip", "attn_prefill.hip", "attn_backward.hip",
           "attn_decode.hip", "attn_decode_drope.hip", "cache.hip"]
CALIB_LIB = os.path.join(HERE, "libdar_calib.so")
CALIB_SOURCES = ["calib.hip"]
HEADERS = ["dar_common.hpp"]
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=" + ARCH,
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _compile(sources, lib, verbose):
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + srcs + [
        "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "warnings generated" not in l)
    if r.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile libdar.so and libdar_calib.so (always recompiles)."""
    _compile(CALIB_SOURCES, CALIB_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
