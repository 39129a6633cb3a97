"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The kernels cannot run under a GPU sanitizer here, so the host-side code is
checked instead: the C ABI's argument checks, shape and size arithmetic and
status strings (tests/sanitize/abi_driver.c against a build of the library
whose host part is instrumented), and the fp64 oracle over seeded inputs and
the edge cases its callers meet (tests/sanitize/oracle_driver.c).  Any
sanitizer report ends that test program with a non-zero status; leaks are reported
too."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "speculative_sampling_verification_softmax_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="3")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{cmd[0]} failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    _run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "spec_oracle.c"), "-o", exe, "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "oracle driver: ok" in r.stdout
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    hipcc, clang = "/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    lib = str(tmp_path / "libspec_sanitized.so")
    # the instrumentation goes to the host pass only (-Xarch_host before each
    # flag); the device code is built as for the library itself
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    _run([hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
          "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "spec_softmax.hip"),
          "-o", lib], timeout=600)
    exe = str(tmp_path / "abi_driver")
    _run([clang, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), lib,
          f"-Wl,-rpath,{tmp_path}", "-o", exe])
    r = _run([exe], env=ENV, timeout=120)
    assert "abi driver: ok" in r.stdout
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-3000:]
