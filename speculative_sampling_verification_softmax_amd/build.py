"""Build libspec_softmax.so (HIP, gfx950) in the package directory.

    python -m speculative_sampling_verification_softmax_amd.build

Compiles csrc/spec_softmax.hip with hipcc for gfx950 only.  Packed fp32
instructions are disabled (-packed-fp32-ops) and floating-point contraction
is off, so every rounding is the one written in the source.  Also builds
libspec_probe.so from csrc/read_ceiling.hip, a streaming-read probe the
benchmark uses to measure this part's read ceiling, and libspec_phases.so, the
same library with the kernels' phase timestamps compiled in
(-DSPEC_PHASE_STAMPS), which only the benchmark's phase mode loads.  Neither is
part of the verify.
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
PHASES_LIB = os.path.join(PKG, "libspec_phases.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libspec_softmax.so)")


def command(out: str = LIB, src: str = SRC, defines: tuple = ()) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", os.path.join(PKG, "csrc"),
            *[f"-D{d}" for d in defines], src, "-o", out]


def _compile_all(jobs: list, verbose: bool) -> None:
    """Runs hipcc for every (src, lib, defines) at once, then moves each
    finished library into place; raises on the first failure."""
    procs = []
    for src, lib, defines in jobs:
        cmd = command(lib + ".tmp", src, defines)
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    # hipcc's host pass warns that it does not know the packed-fp32 feature; ignore that line.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    failed = None
    for lib, p in procs:
        _, stderr = p.communicate()
        err = "\n".join(l for l in stderr.splitlines() if noise not in l)
        if p.returncode != 0:
            failed = failed or f"hipcc failed for {os.path.basename(lib)} ({p.returncode}):\n{err}"
            continue
        if err.strip() and verbose:
            print(err, file=sys.stderr)
        os.replace(lib + ".tmp", lib)
    if failed:
        raise RuntimeError(failed)


def build(verbose: bool = False) -> str:
    """Compile the verify library, the read-ceiling probe and the phase-stamped
    measurement build of the library; returns the library's path."""
    _compile_all([(PROBE_SRC, PROBE_LIB, ()), (SRC, LIB, ()),
                  (SRC, PHASES_LIB, ("SPEC_PHASE_STAMPS",))], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
