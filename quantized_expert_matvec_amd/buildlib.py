"""Build libfmoe.so in-tree with hipcc for gfx950 (MI355X)."""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(_HERE)
SOURCES = ["csrc/kernels.hip", "csrc/api.cpp", "csrc/pack.cpp"]
OUT = os.path.join(_HERE, "libfmoe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-mcode-object-version=5",  # loadable by the HIP runtime bundled with PyTorch
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 VALU instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", *HIPCC_FLAGS, "-I" + os.path.join(ROOT, "include")]
    cmd += [os.path.join(_HERE, s) for s in SOURCES]
    cmd += ["-o", OUT + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if verbose or r.returncode != 0:
        print(" ".join(cmd))
        if out.strip():
            print(out)
    if r.returncode != 0:
        raise RuntimeError("libfmoe build failed")
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
