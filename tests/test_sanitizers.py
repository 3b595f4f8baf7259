"""AddressSanitizer and UndefinedBehaviorSanitizer runs of the CPU-side code
(no GPU needed, nothing launched):

  * the oracle (oracle/oracle.c) with a C driver (tests/sanitize/
    oracle_driver.c) that calls every entry point on small problems whose
    buffers have their exact sizes;
  * the library's host layer (argument and geometry checks, workspace
    planning, status strings, timing switches, the spectral entry points'
    checks, the fixed-point bounds) with a C driver (tests/sanitize/
    abi_driver.c) linked against a build of libtproj whose host code carries
    the sanitizers (the device code is built without them).

A report from either sanitizer aborts the driver with a non-zero status.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
CSRC = os.path.join(ROOT, "back_projection_amd", "csrc")

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (cmd, r.stdout[-3000:], r.stderr[-3000:])
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=gnu11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-static-libasan", "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers missing")
def test_host_layer_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "libtproj_hostsan.so")
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    # sanitizers on the host side only: each -fsanitize= right after -Xarch_host
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                "-Xarch_host", "-g"]
    _run([HIPCC, "--offload-arch=gfx950", "-O0", "-std=c++17", "-fPIC", "-shared", *host_san,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, *sources, "-o", lib,
          "-L/opt/rocm/lib", "-lhipfft", "-Wl,-rpath,/opt/rocm/lib"], timeout=900)
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-std=gnu11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"), "-o", exe,
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"), lib, "-Wl,-rpath," + str(tmp_path), "-lm"])
    r = _run([exe], env=ENV, timeout=300)
    assert "0 failures" in r.stdout
