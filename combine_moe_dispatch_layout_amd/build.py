"""Build libmoe_dispatch.so (the HIP kernels + C ABI) for gfx950, in-tree.

    python -m combine_moe_dispatch_layout_amd.build

Each source is compiled to an object in parallel, then linked into one shared
library next to this file.  Flags: -O3, gfx950 only, and packed-fp32 code
generation disabled (the kernels' fp32 arithmetic is scalar by design).
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libmoe_dispatch.so")
SOURCES = ["api.hip", "layout.hip", "dispatch.hip", "fused.hip", "combine.hip", "probe.hip",
           "noalloc.hip", "planner.cpp"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _obj_dir() -> str:
    d = os.path.join(HERE, "_build")
    os.makedirs(d, exist_ok=True)
    return d


# Build-time tuning macros (for example "-DMOE_CACHED_ROWS_PER_CU=8"); the
# defaults in csrc/moe_internal.h are the measured choices.
EXTRA = os.environ.get("MOE_HIPCC_DEFINES", "").split()


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(_obj_dir(), os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA, f"-I{INCLUDE}", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as pool:
        objs = list(pool.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    exports = os.path.join(CSRC, "exports.map")  # only the moe_* C ABI is exported
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
           f"-Wl,--version-script={exports}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
