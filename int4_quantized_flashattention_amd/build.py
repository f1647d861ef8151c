"""Build the rotattn HIP library (gfx950) in-tree: librotattn.so next to this file.

Usage: python -m int4_quantized_flashattention_amd.build [--jobs N] [--asan]

--asan builds _build/asan/librotattn_asan.so instead: the host code compiled with AddressSanitizer (device
code unchanged; -O1 -g). Load it with ROTATTN_LIBRARY=<path> and the sanitizer runtime preloaded, e.g.
  LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
  ASAN_OPTIONS=detect_leaks=0:verify_asan_link_order=0 ROTATTN_LIBRARY=_build/asan/librotattn_asan.so python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librotattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["prologue.hip", "vquant.hip", "attn_int4.hip", "attn_fp16.hip", "sparse_mask.hip", "rotattn_api.hip"]

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # every rounding step of the prologue is spelled out; no implicit FMA contraction anywhere
    "-ffp-contract=off",
    # no packed-FP32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


ASAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, asan: bool = False) -> str:
    out_dir = os.path.join(BUILD, "asan") if asan else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = [f for f in FLAGS if f != "-O3"] + ASAN_FLAGS if asan else FLAGS
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = True, asan: bool = False) -> str:
    out_dir = os.path.join(BUILD, "asan") if asan else BUILD
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda f: _compile(f, asan), SOURCES))
    lib = os.path.join(out_dir, "librotattn_asan.so") if asan else LIB
    tmp = lib + ".tmp"
    link = ["-Xarch_host", "-fsanitize=address"] if asan else []
    cmd = [HIPCC, "-shared", "--offload-arch=gfx950", "-fPIC", *link, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("--asan", action="store_true", help="host code with AddressSanitizer, into _build/asan/")
    a = ap.parse_args()
    try:
        build(a.jobs, asan=a.asan)
    except RuntimeError as e:
        print(e, file=sys.stderr)
        sys.exit(1)
