"""Build the HIP library liblora_mi355x.so in-tree for gfx950.

    python -m adapter_mlp_amd.build

Every .hip file under csrc/ is compiled with hipcc to an object in _build/
and linked into adapter_mlp_amd/liblora_mi355x.so.  No GPU is needed to build.

    python -m adapter_mlp_amd.build --timing

builds the same sources with -DLORA_BLOCK_TIMING into
adapter_mlp_amd/liblora_mi355x_timing.so: the GEMM kernels then record per-block
clock stamps, read by `bench.py --block-timing` through lora_block_times.

    python -m adapter_mlp_amd.build --phases

builds them with -DLORA_PHASE_TIMING into adapter_mlp_amd/liblora_mi355x_phases.so,
whose GEMM kernels read the shader clock at every phase boundary of one K step
(`bench.py --phase-timing`, through lora_phase_times).  The normal library is
unaffected by either (its GEMM code is the same instruction for instruction).
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
# instrumented variants: name -> (macro, object folder, library)
VARIANTS = {
    "timing": ("LORA_BLOCK_TIMING", os.path.join(PKG, "_build_timing"), os.path.join(PKG, "liblora_mi355x_timing.so")),
    "phases": ("LORA_PHASE_TIMING", os.path.join(PKG, "_build_phases"), os.path.join(PKG, "liblora_mi355x_phases.so")),
}
LIB_TIMING = VARIANTS["timing"][2]
LIB_PHASES = VARIANTS["phases"][2]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU ops are disabled for device code: hipcc would otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I" + INCLUDE, "-I" + CSRC,
          "-Wall", "-Wno-unused-function"] + DEVICE_FLAGS


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, variant=None):
    folder = VARIANTS[variant][1] if variant else BUILD
    obj = os.path.join(folder, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC] + CFLAGS + (["-D" + VARIANTS[variant][0]] if variant else []) + ["-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (p.stdout + p.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if p.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, "\n".join(msgs)))
    return obj, msgs


def build(verbose: bool = False, timing: bool = False, variant: str = None) -> str:
    """Compile and link; returns the path of the shared library (an
    instrumented variant with variant="timing" or "phases"; timing=True is
    variant="timing")."""
    if timing:
        variant = "timing"
    if variant is not None and variant not in VARIANTS:
        raise ValueError(f"unknown build variant {variant!r}")
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(VARIANTS[variant][1] if variant else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda f: _compile(f, variant), srcs))
    objs = []
    for obj, msgs in results:
        objs.append(obj)
        if verbose:
            for m in msgs:
                print(m)
    lib = VARIANTS[variant][2] if variant else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError("link failed:\n" + p.stdout + p.stderr)
    shutil.move(tmp, lib)
    return lib


if __name__ == "__main__":
    v = "timing" if "--timing" in sys.argv else "phases" if "--phases" in sys.argv else None
    print(build(verbose="-v" in sys.argv, variant=v))
