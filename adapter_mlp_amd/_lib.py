"""ctypes mirror of include/lora_mi355x.h and the loader of liblora_mi355x.so.

This module only marshals arguments: every step of the computation runs in
the library's HIP kernels.  Loading fails loudly when the library has not been
built (``python -m adapter_mlp_amd.build``); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblora_mi355x.so")

LORA_OK, LORA_EINVAL, LORA_ESHAPE, LORA_EDTYPE, LORA_EALIGN, LORA_EWORKSPACE, LORA_EUNSUPPORTED, LORA_EDEVICE = range(8)
LORA_F32, LORA_BF16, LORA_BF16_F32LORA = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 32 << 20  # LORA_NOALLOC_SCRATCH_BYTES
LORA_ACT_SWIGLU, LORA_ACT_GEGLU_TANH = 0, 1
ACT_CODES = {"swiglu": LORA_ACT_SWIGLU, "geglu_tanh": LORA_ACT_GEGLU_TANH}
STATUS_NAMES = {0: "LORA_OK", 1: "LORA_EINVAL", 2: "LORA_ESHAPE", 3: "LORA_EDTYPE", 4: "LORA_EALIGN",
                5: "LORA_EWORKSPACE", 6: "LORA_EUNSUPPORTED", 7: "LORA_EDEVICE"}

vp = C.c_void_p
i64 = C.c_int64
i32 = C.c_int32
sz = C.c_size_t


class lora_nf4(C.Structure):
    _fields_ = [("codes", vp), ("q8", vp), ("s2", vp), ("mu", vp), ("rows", i64), ("cols", i64)]


class lora_proj(C.Structure):
    _fields_ = [("W", vp), ("nf4", C.POINTER(lora_nf4)), ("A", vp), ("B", vp), ("scale", C.c_float), ("Wt", vp)]


class lora_gemm_plan(C.Structure):
    _fields_ = [("group", i32), ("ksplit", i32)]


class lora_plan(C.Structure):
    _fields_ = [("gemm", lora_gemm_plan * 2)]


class lora_mlp_desc(C.Structure):
    _fields_ = [("T", i64), ("H", i64), ("I", i64), ("r", i64), ("act", i32), ("dtype", i32),
                ("plan", C.POINTER(lora_plan))]


class lora_mlp_saved(C.Structure):
    _fields_ = [("e", vp), ("g", vp), ("U", vp)]


class lora_mlp_grads(C.Structure):
    _fields_ = [("dA_gate", vp), ("dB_gate", vp), ("dA_up", vp), ("dB_up", vp), ("dA_down", vp), ("dB_down", vp)]


class lora_relu2_mlp_desc(C.Structure):
    _fields_ = [("T", i64), ("H", i64), ("I", i64), ("r", i64), ("dtype", i32), ("reserved", i32),
                ("plan", C.POINTER(lora_plan))]


class lora_relu2_mlp_saved(C.Structure):
    _fields_ = [("u", vp), ("U", vp)]


class lora_relu2_mlp_grads(C.Structure):
    _fields_ = [("dA_up", vp), ("dB_up", vp), ("dA_down", vp), ("dB_down", vp)]


class lora_qkv_desc(C.Structure):
    _fields_ = [("T", i64), ("H", i64), ("Nq", i64), ("Nk", i64), ("Nv", i64), ("r", i64),
                ("dtype", i32), ("reserved", i32), ("plan", C.POINTER(lora_plan))]


class lora_qkv_grads(C.Structure):
    _fields_ = [("dA_q", vp), ("dB_q", vp), ("dA_k", vp), ("dB_k", vp), ("dA_v", vp), ("dB_v", vp)]


class lora_trace_entry(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("launches", i64), ("total_ms", C.c_double)]


class lora_o_desc(C.Structure):
    _fields_ = [("T", i64), ("K", i64), ("N", i64), ("r", i64), ("dtype", i32), ("reserved", i32),
                ("plan", C.POINTER(lora_plan))]


P = C.POINTER
SIGNATURES = {
    "lora_version": (i32, []),
    "lora_strerror": (C.c_char_p, [i32]),
    "lora_last_error": (C.c_char_p, []),
    "lora_nf4_codebook": (None, [P(C.c_float)]),
    "lora_mlp_workspace_size": (i32, [P(lora_mlp_desc), P(sz), P(sz)]),
    "lora_mlp_fwd": (i32, [P(lora_mlp_desc), vp, P(lora_proj), P(lora_proj), P(lora_proj), vp,
                           P(lora_mlp_saved), vp, sz, vp]),
    "lora_mlp_bwd": (i32, [P(lora_mlp_desc), vp, vp, P(lora_mlp_saved), P(lora_proj), P(lora_proj),
                           P(lora_proj), vp, P(lora_mlp_grads), vp, sz, vp]),
    "lora_relu2_mlp_workspace_size": (i32, [P(lora_relu2_mlp_desc), P(sz), P(sz)]),
    "lora_relu2_mlp_fwd": (i32, [P(lora_relu2_mlp_desc), vp, P(lora_proj), P(lora_proj), vp,
                                 P(lora_relu2_mlp_saved), vp, sz, vp]),
    "lora_relu2_mlp_bwd": (i32, [P(lora_relu2_mlp_desc), vp, vp, P(lora_relu2_mlp_saved), P(lora_proj),
                                 P(lora_proj), vp, P(lora_relu2_mlp_grads), vp, sz, vp]),
    "lora_qkv_workspace_size": (i32, [P(lora_qkv_desc), P(sz), P(sz)]),
    "lora_qkv_fwd": (i32, [P(lora_qkv_desc), vp, P(lora_proj), P(lora_proj), P(lora_proj), vp, vp, vp, vp,
                           vp, sz, vp]),
    "lora_qkv_bwd": (i32, [P(lora_qkv_desc), vp, vp, vp, vp, vp, P(lora_proj), P(lora_proj), P(lora_proj),
                           vp, P(lora_qkv_grads), vp, sz, vp]),
    "lora_o_workspace_size": (i32, [P(lora_o_desc), P(sz), P(sz)]),
    "lora_o_fwd": (i32, [P(lora_o_desc), vp, P(lora_proj), vp, vp, vp, sz, vp]),
    "lora_o_bwd": (i32, [P(lora_o_desc), vp, vp, vp, P(lora_proj), vp, vp, vp, vp, sz, vp]),
    "lora_o_fwd_noalloc": (i32, [P(lora_o_desc), vp, P(lora_proj), vp, vp, vp]),
    "lora_nf4_quantize_workspace_size": (i32, [i64, i64, P(sz)]),
    "lora_nf4_quantize": (i32, [vp, i64, i64, i32, vp, vp, vp, vp, vp, sz, vp]),
    "lora_nf4_dequant": (i32, [P(lora_nf4), vp, i32, vp]),
    "lora_nf4_unpack_codes": (i32, [P(lora_nf4), vp, vp]),
    "lora_nf4_gemm_workspace_size": (i32, [i64, i64, i64, i64, i32, P(sz)]),
    "lora_nf4_gemm": (i32, [i64, i32, vp, P(lora_nf4), vp, vp, i64, C.c_float, vp, vp, sz, vp]),
    "lora_trace_begin": (i32, [C.c_char_p]),
    "lora_trace_end": (i32, [P(lora_trace_entry), i32, P(i32)]),
}

_lib = None


class LoraError(RuntimeError):
    def __init__(self, fn, status, detail):
        self.status = status
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}: {detail}")


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m adapter_mlp_amd.build` "
                           "(the package has no non-HIP fallback)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def call(name: str, *args) -> None:
    """Call a status-returning entry point; raise LoraError on failure."""
    lib = load()
    st = getattr(lib, name)(*args)
    if st != LORA_OK:
        raise LoraError(name, st, lib.lora_last_error().decode())
