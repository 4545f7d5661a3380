"""Build libmsa.so (gfx950) in-tree with hipcc.

    python block_sparse_attention_10_amd/build.py

Every HIP translation unit under csrc/ is compiled to an object in
_build/ (not tracked) and linked into block_sparse_attention_10_amd/libmsa.so.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU ops stay disabled for all device code.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
         "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, extra_flags=()) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        src, obj = pair
        out = _run([HIPCC, *FLAGS, *extra_flags, "-c", src, "-o", obj])
        if verbose and out.strip():
            print(out)

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def build_counter_driver(src: str, exe: str) -> str:
    """The torch-free driver of the rocprofv3 counter runs (a measurement
    tool, not part of the library), linked against the built libmsa.so; the
    run path is relative to the executable, so the tree can move."""
    rel = os.path.relpath(PKG, os.path.dirname(os.path.abspath(exe)))
    tmp = exe + ".tmp"
    _run([HIPCC, *FLAGS, src, "-o", tmp, "-L", PKG, "-lmsa", "-Wl,-rpath,$ORIGIN/" + rel])
    os.replace(tmp, exe)
    return exe


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
