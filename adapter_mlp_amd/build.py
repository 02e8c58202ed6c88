"""Build the HIP library liblora_mi355x.so in-tree for gfx950.

    python -m adapter_mlp_amd.build

Every .hip file under csrc/ is compiled with hipcc to an object in _build/
and linked into adapter_mlp_amd/liblora_mi355x.so.  No GPU is needed to build.

    python -m adapter_mlp_amd.build --timing

builds the same sources with -DLORA_BLOCK_TIMING into
adapter_mlp_amd/liblora_mi355x_timing.so: the GEMM kernels then record per-block
clock stamps, read by `bench.py --block-timing` through lora_block_times.  The
normal library is unaffected (its GEMM code is the same instruction for
instruction).
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblora_mi355x.so")
BUILD_TIMING = os.path.join(PKG, "_build_timing")
LIB_TIMING = os.path.join(PKG, "liblora_mi355x_timing.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for device code: hipcc would otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + INCLUDE, "-I" + CSRC,
          "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, timing=False):
    obj = os.path.join(BUILD_TIMING if timing else BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + CFLAGS + (["-DLORA_BLOCK_TIMING"] if timing else []) + ["-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (p.stdout + p.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    return obj, msgs


def build(verbose: bool = False, timing: bool = False) -> str:
    """Compile and link; returns the path of the shared library (the timing
    variant with timing=True)."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_TIMING if timing else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda f: _compile(f, timing), srcs))
    objs = []
    for obj, msgs in results:
        objs.append(obj)
        if verbose:
            for m in msgs:
                print(m)
    lib = LIB_TIMING if timing else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    shutil.move(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timing="--timing" in sys.argv))
