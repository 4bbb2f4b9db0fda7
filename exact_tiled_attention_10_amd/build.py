"""Build libfa.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

Run as ``python -m exact_tiled_attention_10_amd.build`` or call ``build()``.
The library lands next to this file so it travels with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
BUILD_DIR = os.path.join(PKG, "_build")

SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_device.hip", "fa_plan.cpp", "fa_api.cpp"]
# host-only sources of the sanitizer build (no device code; fa_host_stub.cpp
# stands in for the launchers)
ASAN_SOURCES = ["fa_api.cpp", "fa_plan.cpp", "fa_host_stub.cpp"]
ASAN_LIB = os.path.join(BUILD_DIR, "libfa_asan.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 VALU (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # the LDS DMA helper clobbers m0 in inline assembly on purpose (fa_common.h)
    "-Wno-inline-asm",
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; libfa.so needs ROCm's hipcc")
    return exe


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libfa.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc, "-O2", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
                   "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    link = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}")
    os.replace(tmp, LIB)
    return LIB


def build_host_asan(verbose: bool = False) -> str:
    """Build the C ABI layer alone (argument checks, size queries, plans) as
    a host library under AddressSanitizer and UBSan, with the kernel
    launchers stubbed out: for exercising the boundary on a CPU-only machine.
    Returns the library's path; load it with the ASan runtime preloaded."""
    gxx = shutil.which("g++")
    if gxx is None:
        raise RuntimeError("g++ not found; the sanitizer build needs it")
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = ASAN_LIB + ".tmp"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in ASAN_SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{r.stdout}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_host_asan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
