"""Build step for libflce.so (gfx950): hipcc compiles the HIP kernels and the C-ABI host code in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
# FLCE_LIB selects another build of the library (e.g. a different pipeline geometry); build() and
# ensure_built() always refer to the in-tree default.
DEFAULT_LIB = os.path.join(PKG, "libflce.so")
LIB = os.environ.get("FLCE_LIB", DEFAULT_LIB)
SOURCES = ["flce_kernels.hip", "flce_api.cpp"]

# Packed fp32 VALU forms stay off: ordinary float code is left to scalar VALU instructions.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libflce.so)")


def build(verbose: bool = False) -> str:
    """Compile libflce.so for gfx950 into the package directory and return its path."""
    tmp = DEFAULT_LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(tmp, DEFAULT_LIB)
    return DEFAULT_LIB


CALIB_LIB = os.path.join(PKG, "libflce_calib.so")


def build_calib(verbose: bool = False) -> str:
    """Compile the benchmark's peak-calibration library (MFMA-only loop, device copy) for gfx950."""
    tmp = CALIB_LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", INCLUDE, os.path.join(CSRC, "flce_calib.hip"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(tmp, CALIB_LIB)
    return CALIB_LIB


EXAMPLE_SRC = os.path.join(PKG, "examples", "flce_from_c.c")
EXAMPLE_BIN = os.path.join(PKG, "examples", "flce_from_c")


def build_c_example(verbose: bool = False) -> str:
    """Compile the plain C99 caller of the library (gcc; HIP runtime C API for device memory)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, EXAMPLE_SRC,
           "-L", PKG, "-lflce", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/..", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", EXAMPLE_BIN + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr[-8000:]}")
    os.replace(EXAMPLE_BIN + ".tmp", EXAMPLE_BIN)
    return EXAMPLE_BIN


def ensure_built() -> str:
    """Return the library path, building it only if no library exists yet."""
    if not os.path.exists(LIB):
        if LIB != DEFAULT_LIB:
            raise FileNotFoundError(f"FLCE_LIB={LIB} does not exist")
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
