"""Build libbimamba.so in-tree with hipcc for gfx950.

    python -m bidirectional_mamba_selective_amd.build

Compiles every source under csrc/ into one shared library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbimamba.so")
ARCH = "gfx950"

# Packed fp32 instructions stay disabled for all device code.
HIPFLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbimamba.so")


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPFLAGS, *extra_flags, "-I", os.path.join(os.path.dirname(PKG), "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that warning is harmless
    noise = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
