"""Build libbimamba.so (and the benchmark's libbimamba_micro.so) in-tree with hipcc for gfx950.

    python -m bidirectional_mamba_selective_amd.build
    python -m bidirectional_mamba_selective_amd.build --asan-host

Compiles every source under csrc/ into one shared library next to this file,
and micro/micro_kernels.hip (the microbenchmarks behind the reported rooflines)
into a second one.  --asan-host instead writes libbimamba_asan.so: the same
sources with AddressSanitizer on the host code only (argument checking, plans,
launches; device code is built as usual), for the ABI tests on the CPU:

    LD_PRELOAD=$(gcc -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
        python -m pytest tests/test_abi.py -m "not gpu" -p no:cacheprovider \
        --bimamba-lib bidirectional_mamba_selective_amd/libbimamba_asan.so
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbimamba.so")
MICRO_SRC = os.path.join(PKG, "micro", "micro_kernels.hip")
MICRO_LIB = os.path.join(PKG, "libbimamba_micro.so")
ASAN_LIB = os.path.join(PKG, "libbimamba_asan.so")
# AddressSanitizer for the host pass only (each -fsanitize= behind -Xarch_host)
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
ARCH = "gfx950"

# Packed fp32 instructions stay disabled for all device code.
HIPFLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Per-source device code generation.  The scan kernels issue faster when the machine scheduler orders their
# instructions for instruction-level parallelism (measured on MI355X at L = 65536, two runs each: the tied
# call 1.632 -> 1.609 ms, untied directions 2.685 -> 2.592 ms, identical output bits); the Mamba-2 kernels
# keep the default order (with it their fused one-direction layers took 2.43 instead of 2.37 ms).
SOURCE_FLAGS = {"scan_kernels.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libbimamba.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that warning is harmless
    noise = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(noise))
    if verbose and noise:
        print("\n".join(noise))


def _compile(srcs, lib, verbose, extra_flags=()):
    """Each source to an object with its own flags (SOURCE_FLAGS), then one shared library."""
    tmp = lib + ".tmp"
    inc = os.path.join(os.path.dirname(PKG), "include")
    os.makedirs(os.path.join(PKG, "_build"), exist_ok=True)
    objdir = tempfile.mkdtemp(prefix="objs_", dir=os.path.join(PKG, "_build"))
    try:
        objs = []
        for src in srcs:
            obj = os.path.join(objdir, os.path.basename(src) + ".o")
            _run([hipcc(), *HIPFLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []), *extra_flags, "-I", inc, "-c", src,
                  "-o", obj], verbose)
            objs.append(obj)
        _run([hipcc(), "-fPIC", "-shared", *extra_flags, *objs, "-o", tmp], verbose)
    finally:
        shutil.rmtree(os.path.join(PKG, "_build"), ignore_errors=True)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile both libraries; returns the path of libbimamba.so."""
    lib = _compile(sources(), LIB, verbose, extra_flags)
    _compile([MICRO_SRC], MICRO_LIB, verbose, extra_flags)
    return lib


def build_asan_host(verbose: bool = False) -> str:
    """The library with AddressSanitizer on its host code, as libbimamba_asan.so."""
    return _compile(sources(), ASAN_LIB, verbose, ASAN_HOST_FLAGS)


if __name__ == "__main__":
    if "--asan-host" in sys.argv:
        print(build_asan_host(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
