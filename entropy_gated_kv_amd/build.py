"""Build libec.so for gfx950 with hipcc (in-tree, next to this file).

Every HIP source compiles to an object in _build/ and the objects link into
entropy_gated_kv_amd/libec.so.  Always rebuilds (the build check compiles
every time it is asked to).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libec.so")

SOURCES = ["entropy.hip", "select.hip", "glue.hip", "gemm.hip", "attention.hip", "drift.hip",
           "noalloc.hip", "ec_validate.cpp", "ec_api.cpp"]
ARCH = "gfx950"
# Packed FP32 (v_pk_fma/mul/add_f32) is disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC]
# Per-source device options: MFMA results in ordinary VGPRs.  attention.hip:
# the accumulator-register form makes the compiler copy the output tile between
# register files on every kv tile.  gemm.hip: it lowers the skinny kernels'
# register count (the 96-row instance fits three waves per SIMD instead of two).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA = {"attention.hip": _VGPR_FORM, "gemm.hip": _VGPR_FORM}


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = ([_hipcc()] + COMMON + DEVICE_FLAGS + EXTRA.get(src, []) + lang +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


DRIVER_SRC = os.path.join(ROOT, "tests", "c_abi_driver.cpp")
DRIVER = os.path.join(ROOT, "tests", "c_abi_driver")


def build_c_driver() -> str:
    """The test suite's plain C++ user of libec.so (host code only, so the
    host compiler builds it against include/ec.h and the HIP runtime); it
    finds libec.so next to the package through its run path."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [gxx, "-std=c++17", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE,
           "-I", os.path.join(rocm, "include"), DRIVER_SRC, "-o", DRIVER + ".tmp",
           "-L", PKG, "-lec", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../entropy_gated_kv_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"driver build failed\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(DRIVER + ".tmp", DRIVER)
    return DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_driver())
