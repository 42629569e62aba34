"""Build libfmoe.so in-tree with hipcc for gfx950 (MI355X).

Each translation unit compiles to an object under _build/ (in parallel), then
hipcc links the shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
SOURCES = ["csrc/kernels_q4.hip", "csrc/kernels_q2.hip", "csrc/kernels.hip", "csrc/kernels_forms.hip", "csrc/scratch.hip", "csrc/tier_kernels.hip", "csrc/api.cpp",
           "csrc/pack.cpp"]
OUT = os.path.join(_HERE, "libfmoe.so")
BUILD_DIR = os.path.join(ROOT, "_build", "fmoe")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",  # loadable by the HIP runtime bundled with PyTorch
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 VALU instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        if out.strip():
            print(out)
    if r.returncode != 0:
        raise RuntimeError(f"libfmoe build failed: {' '.join(cmd)}")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = "-I" + os.path.join(ROOT, "include")
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append(["hipcc", *HIPCC_FLAGS, inc, *lang, "-c", os.path.join(_HERE, src), "-o", obj])
        objs.append(obj)
    workers = min(len(cmds), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", OUT + ".tmp"], verbose)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
