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
           "quantize_fp8.hip", "attn_noalloc.hip"]

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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=6)
    args = ap.parse_args(argv)
    build(args.jobs, verbose=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
