"""Build libspec_softmax.so (HIP, gfx950) in the package directory.

    python -m speculative_sampling_verification_softmax_amd.build

Compiles csrc/spec_softmax.hip with hipcc for gfx950 only.  Packed fp32
instructions are disabled (-packed-fp32-ops) and floating-point contraction
is off, so every rounding is the one written in the source.  Also builds
libspec_probe.so from csrc/read_ceiling.hip, a streaming-read probe the
benchmark uses to measure this part's read ceiling (not part of the verify).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "spec_softmax.hip")
LIB = os.path.join(PKG, "libspec_softmax.so")
PROBE_SRC = os.path.join(PKG, "csrc", "read_ceiling.hip")
PROBE_LIB = os.path.join(PKG, "libspec_probe.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libspec_softmax.so)")


def command(out: str = LIB, src: str = SRC) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"),
            src, "-o", out]


def _compile(src: str, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = command(tmp, src)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; ignore that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile the verify library and the read-ceiling probe; returns the library's path."""
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    return _compile(SRC, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
