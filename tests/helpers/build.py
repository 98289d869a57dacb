"""Builds the GPU test helper programs in tests/helpers/ (hipcc, gfx950) into
tests/helpers/_build/.  Called by __graft_entry__.build(); runs without a GPU."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "_build")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> list:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OUT, exist_ok=True)
    built = []
    for src in sorted(glob.glob(os.path.join(HERE, "*.hip"))):
        exe = os.path.join(OUT, os.path.splitext(os.path.basename(src))[0])
        subprocess.run([hipcc, *FLAGS, src, "-o", exe + ".tmp"], check=True)
        os.replace(exe + ".tmp", exe)
        built.append(exe)
    return built


if __name__ == "__main__":
    print("\n".join(build()))
