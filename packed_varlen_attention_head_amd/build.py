"""Builds libh3a.so (gfx950) in-tree with hipcc.

    python -m packed_varlen_attention_head_amd.build [--jobs N]

Objects go to _build/ at the repository root; the shared library is written
next to this file, where the Python binding loads it from.
"""
from __future__ import annotations

import argparse
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
LIB = os.path.join(PKG, "libh3a.so")

SOURCES = ["api.cpp", "planner.cpp", "rope_table.hip", "qk_norm_rope.hip", "attn_fwd_bf16.hip", "attn_fwd_f32.hip",
           "quantize_fp8.hip", "quantize_i8.hip", "attn_noalloc.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fno-strict-aliasing", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libh3a.so)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc(), *COMMON_FLAGS, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature: harmless.
    err = "\n".join(line for line in r.stderr.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 6, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libh3a.so failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host code only (the C ABI's validation, plan cache and planner): compiled
# with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, linked with
# the ordinary kernel objects.  The GPU code is never sanitised.
HOST_SOURCES = ["api.cpp", "planner.cpp"]
SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libh3a_san.so")
SAN_FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
             "-I", INCLUDE, "-I", CSRC]


def build_sanitized(jobs: int = 6, verbose: bool = False) -> str:
    """libh3a_san.so: api.cpp and planner.cpp built by g++ with ASan + UBSan, the
    HIP sources as in build().  Load it with H3A_LIBRARY and LD_PRELOAD of
    g++'s libasan (`g++ -print-file-name=libasan.so`)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    kernels = [s for s in SOURCES if s not in HOST_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        kobjs = list(ex.map(_compile, kernels))
    hobjs = []
    for src in HOST_SOURCES:
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        cmd = ["g++", *SAN_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} (sanitizers) failed:\n{' '.join(cmd)}\n{r.stderr}")
        hobjs.append(obj)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *hobjs, *kobjs, "-lasan", "-lubsan",
           "-o", SAN_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {SAN_LIB} failed:\n{' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=6)
    ap.add_argument("--sanitize", action="store_true",
                    help="build _build/san/libh3a_san.so (host code under ASan + UBSan) instead")
    args = ap.parse_args(argv)
    if args.sanitize:
        build_sanitized(args.jobs, verbose=True)
    else:
        build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
