"""Build libdsa.so (HIP, gfx950) in-tree with hipcc.

Every ``csrc/*.hip`` file and ``csrc/abi.cpp`` are compiled to objects in
parallel and linked into ``sparse_attention_11_amd/libdsa.so``; the same
sources compiled with ``-DDSA_DEBUG`` (device-side checks, include/dsa.h)
give ``libdsa_debug.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdsa.so")
BUILD_DIR = os.path.join(PKG, "_build")
DEBUG_OUT = os.path.join(PKG, "libdsa_debug.so")
DEBUG_BUILD_DIR = os.path.join(PKG, "_build_debug")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
          # packed fp32 VALU forms are kept out of every kernel
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # multiply-adds are fused only within one source expression, never by
          # the backend across statements: rounding then follows the source, and
          # the checking build (whose extra branches regroup the code) computes
          # the same bits as the release build
          "-ffp-contract=on",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, build_dir: str, extra: list) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, debug: bool = False) -> str:
    out, build_dir = (DEBUG_OUT, DEBUG_BUILD_DIR) if debug else (OUT, BUILD_DIR)
    extra = ["-DDSA_DEBUG"] if debug else []
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "abi.cpp")]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    nums = [a for a in sys.argv[1:] if not a.startswith("-")]
    jobs = int(nums[0]) if nums else 8
    print(build(jobs))
    if "--no-debug" not in sys.argv:
        print(build(jobs, debug=True))
