"""Compile libqsa.so for gfx950 (cross-compiles without a GPU).

The HIP sources in csrc/ (*.hip: kernels and their launchers) go through
hipcc; the host side (*.cpp: validation, workspace layout, launch chains,
accounting) is plain C++ and goes through the host compiler alone, which is
what keeps it free of HIP types and buildable under the sanitizers."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqsa.so")
BUILD = os.path.join(ROOT, "_build", "qsa")

ARCH = "gfx950"
# -ffp-contract=off: every fused multiply-add in the kernels is written out,
#   so the score order is exactly the documented one.
# -fno-gpu-flush-denormals-to-zero: IEEE single with denormals kept.
# -Xclang -target-feature -Xclang -packed-fp32-ops: no packed FP32 (v_pk_*)
#   instructions are generated.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
CXXFLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra",
            "-I", INCLUDE, "-I", CSRC]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libqsa.so")
    return exe


def cxx():
    return shutil.which("g++") or "c++"


def sources(ext):
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(ext))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc(), *HIPFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [cxx(), *CXXFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources(".hip") + sources(".cpp")
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
