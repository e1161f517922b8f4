"""Builds libvk.so in-tree for gfx950 (hipcc for the kernels, g++ for host code).

Usage: python -m bit_ternary_attention_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvk.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

ARCH = "gfx950"
# packed fp32 VALU forms are disabled: the compiler would otherwise form them from float code
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result", "-I" + INCLUDE, "-I" + CSRC]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra",
             "-D__HIP_PLATFORM_AMD__", "-I" + INCLUDE, "-I" + CSRC, "-I" + os.path.join(ROCM, "include")]

# (object name, source, extra flags).  The decode kernels never produce or consume NaN (masked
# scores are -inf), so float max needs no NaN quieting (otherwise each fmaxf operand is
# canonicalised first); their source is compiled once per head dim, in parallel.
HIP_UNITS = [("vk_write", "vk_write.hip", []),
             ("vk_decode_d128", "vk_decode.hip", ["-fno-honor-nans", "-DVK_DECODE_DIM=128"]),
             ("vk_decode_d64", "vk_decode.hip", ["-fno-honor-nans", "-DVK_DECODE_DIM=64"]),
             ("vk_retier", "vk_retier.hip", [])]
CXX_SOURCES = ["host_state.cpp", "vk_api.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build_library(verbose: bool = False) -> str:
    """Compiles every source and links libvk.so; returns its path."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for name, src, extra in HIP_UNITS:
        obj = os.path.join(BUILD, name + ".o")
        jobs.append([hipcc, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs,
          "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")], verbose)
    os.replace(tmp, LIB)
    return LIB


def asm(unit: str, out: str) -> None:
    """Writes the gfx950 assembly of one compile unit (a name of HIP_UNITS), for inspection."""
    hipcc = shutil.which("hipcc") or os.path.join(ROCM, "bin", "hipcc")
    name, src, extra = next(u for u in HIP_UNITS if u[0] == unit)
    _run([hipcc, *HIP_FLAGS, *extra, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out], True)


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
