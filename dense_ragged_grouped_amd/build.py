"""Build step: compile the gfx950 HIP kernels and the C ABI into libdrgg.so.

    python -m dense_ragged_grouped_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The library is written next to
this file (in-tree) so that it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdrgg.so")
SOURCES = ["api.cpp", "kernels.hip"]
ARCH = os.environ.get("DRGG_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # hardware FP32 atomic add for the split-tile sums
    "-munsafe-fp-atomics",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, save_temps_dir: str | None = None) -> str:
    objs = []
    tmpdir = os.path.join(HERE, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = ["hipcc", *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps_dir and src.endswith(".hip"):
            cmd += ["-save-temps=obj"]
            obj_dir = save_temps_dir
            os.makedirs(obj_dir, exist_ok=True)
            cmd[-1] = os.path.join(obj_dir, os.path.basename(obj))
            obj = cmd[-1]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
