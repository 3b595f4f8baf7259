"""Build libtproj.so (gfx950) in-tree with hipcc, and the measurement probes
(libtproj_probes.so, bench.py --peaks)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtproj.so")
PROBES_SRC = os.path.join(PKG, "probes", "probes.hip")
PROBES_LIB = os.path.join(PKG, "libtproj_probes.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed FP32 instructions stay off (v_pk_* FP32 forms are not used)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-parameter",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _hipcc(srcs, out, verbose, libs=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp, *libs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # the host pass does not know this gfx950 feature flag
    errs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip())
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs:
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _hipcc([PROBES_SRC], PROBES_LIB, verbose)
    # hipFFT serves the FFT steps of the spectral front and back ends
    return _hipcc(sources(), LIB, verbose, libs=("-L/opt/rocm/lib", "-lhipfft", "-Wl,-rpath,/opt/rocm/lib"))


if __name__ == "__main__":
    print(build(verbose=True))
