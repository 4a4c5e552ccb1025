"""Build libmxfp4_moe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m mxfp4_mixture_experts_amd.build_lib   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmxfp4_moe.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["route_group.hip", "expert_gemv.hip", "expert_gemm.hip", "combine.hip", "dequantize.hip", "router.hip", "capi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def _flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # no packed-fp32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-result",
    ]


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
        if verbose and res.stderr.strip():
            print(res.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


SANITIZED_LIB = os.path.join(BUILD_DIR, "libmxfp4_moe_hostsan.so")


def build_host_sanitized() -> str:
    """The same library with its host-side C ABI layer (capi.cpp) compiled by g++
    under AddressSanitizer and UndefinedBehaviorSanitizer, linked with the kernel
    objects of build().  For the ABI tests on a host without a GPU: they load it
    (MXFP4_MOE_LIB) with the sanitizer runtimes preloaded.  Returns its path."""
    objs = [os.path.join(BUILD_DIR, src + ".o") for src in SOURCES if src.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build()
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    obj = os.path.join(BUILD_DIR, "capi.hostsan.o")
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    steps = [
        ["g++", "-std=c++17", "-O1", "-g", "-fPIC", *san, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
         "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "capi.cpp"), "-o", obj],
        ["g++", "-shared", *san, "-o", SANITIZED_LIB, obj, *objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
         f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"],
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"sanitized build failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose=True))
