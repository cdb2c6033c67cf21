"""Build libeqlinear.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m group_wise_dft_amd.build`` or ``build_library()``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libeqlinear.so")
SOURCES = ["eqlinear_api.hip", "eqlinear_kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def build_library(extra_flags=None, out: str = LIB, verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + list(extra_flags or []) + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag; that
    # warning is expected and dropped, anything else is shown.
    out_lines = [l for l in r.stdout.splitlines()
                 if "packed-fp32-ops" not in l and "warnings generated" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(out_lines))
    if out_lines and verbose:
        print("\n".join(out_lines))
    # Every kernel launched by the host code must have its stub in the
    # library: an undefined one only shows up at load time otherwise.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], stdout=subprocess.PIPE, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "eqk" in l]
    if nm.returncode != 0 or missing:
        os.unlink(tmp)
        raise RuntimeError("libeqlinear.so has undefined internal symbols: %s" % missing[:4])
    os.replace(tmp, out)
    return out


PEAKS_LIB = os.path.join(PKG, "libeqlinear_peaks.so")


def build_peaks(out: str = PEAKS_LIB, verbose: bool = False) -> str:
    """Compile the microbenchmarks of achievable MI355X rates (bench.py --peaks)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, "peaks.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(sys.argv[1:], verbose=True))
    print(build_peaks(verbose=True))
