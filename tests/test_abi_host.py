"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every function the header declares, and rejects
bad arguments with the documented status before touching the GPU (every
check here fails validation, so nothing is enqueued).
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora_mi355x.h")


@pytest.fixture(scope="module")
def L():
    from adapter_mlp_amd import _lib

    _lib.load()
    return _lib


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert len(names) >= 19
    lib = L.load()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(L.SIGNATURES), "binding signatures out of sync with the header"


def test_version_and_strerror(L):
    lib = L.load()
    assert lib.lora_version() == 3
    for s in range(8):
        assert lib.lora_strerror(s)
    assert lib.lora_strerror(0) == b"success"


def test_codebook_matches_oracle_table(L):
    from oracle.nf4 import NF4_LEVELS

    buf = (C.c_float * 16)()
    L.load().lora_nf4_codebook(buf)
    got = np.array(list(buf), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), NF4_LEVELS.view(np.uint32))


def _status(L, name, *args):
    lib = L.load()
    return getattr(lib, name)(*args)


FAKE = 1 << 20  # 16-byte aligned non-NULL address; never dereferenced (validation fails first)


def _proj(L, W=FAKE, A=FAKE, B=FAKE, scale=2.0, nf4=None):
    p = L.lora_proj()
    p.W, p.A, p.B, p.scale = W, A, B, scale
    if nf4 is not None:
        p.nf4 = C.pointer(nf4)
    return p


def test_mlp_validation_statuses(L):
    sz = C.c_size_t
    f, b = sz(), sz()
    d = L.lora_mlp_desc(128, 256, 720, 16, 0, L.LORA_BF16)
    assert _status(L, "lora_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_ESHAPE  # 720 % 64
    d = L.lora_mlp_desc(128, 256, 768, 16, 0, L.LORA_BF16)
    assert _status(L, "lora_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_OK
    assert f.value > 0 and b.value > 0
    d32 = L.lora_mlp_desc(128, 256, 720, 8, 0, L.LORA_F32)
    assert _status(L, "lora_mlp_workspace_size", C.byref(d32), C.byref(f), C.byref(b)) == L.LORA_OK
    bad = [
        (L.lora_mlp_desc(128, 256, 768, 16, 7, L.LORA_BF16), L.LORA_EINVAL),  # activation
        (L.lora_mlp_desc(128, 256, 768, 16, 0, 9), L.LORA_EDTYPE),
        (L.lora_mlp_desc(-1, 256, 768, 16, 0, L.LORA_BF16), L.LORA_ESHAPE),
        (L.lora_mlp_desc(128, 0, 768, 16, 0, L.LORA_BF16), L.LORA_ESHAPE),
        (L.lora_mlp_desc(128, 256, 768, 12, 0, L.LORA_BF16), L.LORA_ESHAPE),  # r % 8
        (L.lora_mlp_desc(128, 256, 768, 40, 0, L.LORA_BF16), L.LORA_ESHAPE),  # 2r > 64
        (L.lora_mlp_desc(128, 256, 768, 0, 0, L.LORA_F32), L.LORA_ESHAPE),
    ]
    for desc, want in bad:
        assert _status(L, "lora_mlp_workspace_size", C.byref(desc), C.byref(f), C.byref(b)) == want


def test_mlp_fwd_rejects_before_enqueue(L):
    d = L.lora_mlp_desc(128, 256, 768, 16, 0, L.LORA_BF16)
    f, b = C.c_size_t(), C.c_size_t()
    _status(L, "lora_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    sv = L.lora_mlp_saved(FAKE, FAKE, FAKE)
    g, u, dn = _proj(L), _proj(L), _proj(L)

    def fwd(X=FAKE, Y=FAKE * 2, saved=sv, gate=g, ws=FAKE, nbytes=f.value):
        return _status(L, "lora_mlp_fwd", C.byref(d), X, C.byref(gate), C.byref(u), C.byref(dn), Y,
                       C.byref(saved), ws, nbytes, None)

    assert fwd(X=None) == L.LORA_EINVAL
    assert fwd(X=FAKE + 2) == L.LORA_EALIGN
    assert fwd(nbytes=f.value - 1) == L.LORA_EWORKSPACE
    assert fwd(ws=None) == L.LORA_EWORKSPACE
    assert fwd(gate=_proj(L, W=None)) == L.LORA_EINVAL  # neither W nor nf4
    assert fwd(gate=_proj(L, scale=float("nan"))) == L.LORA_EINVAL
    assert fwd(saved=L.lora_mlp_saved(FAKE, None, FAKE)) == L.LORA_EINVAL
    assert fwd(Y=FAKE) == L.LORA_EUNSUPPORTED  # Y aliases X
    assert b"alias" in L.load().lora_last_error()


def test_nf4_validation(L):
    nbytes = C.c_size_t()
    assert _status(L, "lora_nf4_quantize_workspace_size", 64, 256, C.byref(nbytes)) == L.LORA_OK
    assert _status(L, "lora_nf4_quantize_workspace_size", 64, 200, C.byref(nbytes)) == L.LORA_ESHAPE
    q = L.lora_nf4(FAKE, FAKE, FAKE, FAKE, 256, 768)
    # NF4 base with fp32 compute is unsupported
    d = L.lora_o_desc(64, 256, 768, 8, L.LORA_F32, 0)
    f, b = C.c_size_t(), C.c_size_t()
    _status(L, "lora_o_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    o = _proj(L, W=None, nf4=q)
    st = _status(L, "lora_o_fwd", C.byref(d), FAKE, C.byref(o), FAKE * 2, FAKE * 3, FAKE * 4, f.value, None)
    assert st == L.LORA_EUNSUPPORTED
    # shape mismatch between descriptor and NF4 weight
    d16 = L.lora_o_desc(64, 256, 1024, 16, L.LORA_BF16, 0)
    _status(L, "lora_o_workspace_size", C.byref(d16), C.byref(f), C.byref(b))
    st = _status(L, "lora_o_fwd", C.byref(d16), FAKE, C.byref(o), FAKE * 2, FAKE * 3, FAKE * 4, f.value, None)
    assert st == L.LORA_ESHAPE
    # numel not a multiple of 64 * 256
    q2 = L.lora_nf4(FAKE, FAKE, FAKE, FAKE, 64, 64)
    st = _status(L, "lora_nf4_dequant", C.byref(q2), FAKE, L.LORA_BF16, None)
    assert st == L.LORA_ESHAPE
    st = _status(L, "lora_nf4_gemm_workspace_size", 64, 256, 768, 16, 2, C.byref(nbytes))
    assert st == L.LORA_EINVAL  # trans must be 0/1
    # operands of 2 GiB or more (32-bit offsets): the activation [T, max(rows, cols)]
    # and the weight, in the query and in the call itself
    for trans in (0, 1):
        st = _status(L, "lora_nf4_gemm_workspace_size", 1 << 20, 256, 1024, 16, trans, C.byref(nbytes))
        assert st == L.LORA_ESHAPE
        assert _status(L, "lora_nf4_gemm_workspace_size", 64, 1 << 15, 1 << 15, 0, trans, C.byref(nbytes)) == L.LORA_ESHAPE
        assert _status(L, "lora_nf4_gemm_workspace_size", (1 << 20) - 16, 256, 1024, 16, trans,
                       C.byref(nbytes)) == L.LORA_OK
    qbig = L.lora_nf4(FAKE, FAKE, FAKE, FAKE, 256, 1024)
    st = _status(L, "lora_nf4_gemm", 1 << 20, 0, FAKE, C.byref(qbig), None, None, 0, C.c_float(0.0), FAKE * 2,
                 FAKE * 3, 1 << 40, None)
    assert st == L.LORA_ESHAPE


def test_qkv_o_validation(L):
    f, b = C.c_size_t(), C.c_size_t()
    d = L.lora_qkv_desc(100, 4096, 4096, 1024, 1024, 16, L.LORA_BF16, 0)
    assert _status(L, "lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_OK
    d = L.lora_qkv_desc(100, 4096, 4096, 1024, 1024, 24, L.LORA_BF16, 0)  # 3r = 72 > 64
    assert _status(L, "lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_ESHAPE
    d = L.lora_qkv_desc(100, 4096, 4096, 1024, 1024, 16, L.LORA_BF16, 1)
    assert _status(L, "lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_EINVAL
    d = L.lora_o_desc(0, 4096, 4096, 16, L.LORA_BF16, 0)
    assert _status(L, "lora_o_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_OK
    # every operand below 2 GiB: V [T, Nv] with Nv the widest width decides it
    d = L.lora_qkv_desc(65536, 4096, 4096, 1024, 16384, 16, L.LORA_BF16, 0)  # V: 2 GiB
    assert _status(L, "lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_ESHAPE
    d = L.lora_qkv_desc(65535, 4096, 4096, 1024, 16384, 16, L.LORA_BF16, 0)
    assert _status(L, "lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_OK
    d = L.lora_qkv_desc(64, 4096, 64, 64, 262144, 16, L.LORA_BF16, 0)  # W_v [4096, 262144]: 2 GiB
    assert _status(L, "lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b)) == L.LORA_ESHAPE


def test_binding_fails_loudly_without_library(tmp_path):
    from adapter_mlp_amd import _lib

    with pytest.raises(RuntimeError, match="build it"):
        _load_fresh(str(tmp_path / "missing.so"))


def _load_fresh(path):
    from adapter_mlp_amd import _lib

    saved = _lib._lib
    _lib._lib = None
    try:
        return _lib.load(path)
    finally:
        _lib._lib = saved


def test_fp32_lora_mode_workspace_and_dtype_rules(L):
    """LORA_BF16_F32LORA (fp32 adapters and adapter gradients, bf16 otherwise)
    has the bf16 shape rules, and each workspace grows by the bf16 casts of
    the adapters (each cast 256-byte aligned)."""
    sz = C.c_size_t
    T, H, I, r = 300, 256, 768, 16
    fb, bb, ff, bf = sz(), sz(), sz(), sz()
    d = L.lora_mlp_desc(T, H, I, r, 0, L.LORA_BF16)
    assert _status(L, "lora_mlp_workspace_size", C.byref(d), C.byref(fb), C.byref(bb)) == L.LORA_OK
    d2 = L.lora_mlp_desc(T, H, I, r, 0, L.LORA_BF16_F32LORA)
    assert _status(L, "lora_mlp_workspace_size", C.byref(d2), C.byref(ff), C.byref(bf)) == L.LORA_OK
    cast = 3 * (H * r * 2 + r * I * 2)  # every piece here is already a multiple of 256 bytes
    assert ff.value - fb.value == cast and bf.value - bb.value == cast
    bad = L.lora_mlp_desc(T, H, 720, r, 0, L.LORA_BF16_F32LORA)  # bf16 rule: widths % 64
    assert _status(L, "lora_mlp_workspace_size", C.byref(bad), C.byref(ff), C.byref(bf)) == L.LORA_ESHAPE
    dq = L.lora_qkv_desc(T, H, 256, 128, 64, r, L.LORA_BF16_F32LORA, 0)
    assert _status(L, "lora_qkv_workspace_size", C.byref(dq), C.byref(ff), C.byref(bf)) == L.LORA_OK
    do = L.lora_o_desc(T, 256, 512, r, L.LORA_BF16_F32LORA, 0)
    assert _status(L, "lora_o_workspace_size", C.byref(do), C.byref(ff), C.byref(bf)) == L.LORA_OK
    # the NF4 format calls take a tensor dtype, not a mode
    nbytes = sz()
    assert _status(L, "lora_nf4_quantize_workspace_size", 256, 256, C.byref(nbytes)) == L.LORA_OK
    assert _status(L, "lora_nf4_quantize", FAKE, 256, 256, L.LORA_BF16_F32LORA, FAKE, FAKE, FAKE, FAKE, FAKE,
                   nbytes.value, None) == L.LORA_EDTYPE


def test_binding_picks_fp32_lora_mode_from_adapter_dtype():
    import torch

    import adapter_mlp_amd as lm
    from adapter_mlp_amd import _lib

    X = torch.zeros(4, 64, dtype=torch.bfloat16)
    p32 = lm.Proj(A=torch.zeros(64, 8), B=torch.zeros(8, 64), scale=1.0, W=torch.zeros(64, 64, dtype=torch.bfloat16))
    p16 = lm.Proj(A=torch.zeros(64, 8, dtype=torch.bfloat16), B=torch.zeros(8, 64, dtype=torch.bfloat16), scale=1.0,
                  W=torch.zeros(64, 64, dtype=torch.bfloat16))
    assert lm._call_dtype(X, (p32,)) == _lib.LORA_BF16_F32LORA
    assert lm._call_dtype(X, (p16,)) == _lib.LORA_BF16
    with pytest.raises(ValueError):
        lm._call_dtype(X, (p32, p16))  # mixed adapter dtypes
    with pytest.raises(ValueError):
        lm._call_dtype(X.float(), (p16,))  # bf16 adapters with fp32 inputs


def test_relu2_mlp_validation(L):
    sz = C.c_size_t
    f, b = sz(), sz()
    ok = L.lora_relu2_mlp_desc(300, 256, 768, 64, L.LORA_BF16, 0)  # r = 64: one adapter per input
    assert _status(L, "lora_relu2_mlp_workspace_size", C.byref(ok), C.byref(f), C.byref(b)) == L.LORA_OK
    assert f.value > 0 and b.value > 0
    bad = [
        (L.lora_relu2_mlp_desc(300, 256, 720, 16, L.LORA_BF16, 0), L.LORA_ESHAPE),  # 720 % 64
        (L.lora_relu2_mlp_desc(300, 256, 768, 72, L.LORA_BF16, 0), L.LORA_ESHAPE),  # r > 64
        (L.lora_relu2_mlp_desc(300, 256, 768, 16, L.LORA_BF16, 1), L.LORA_EINVAL),  # reserved
        (L.lora_relu2_mlp_desc(-1, 256, 768, 16, L.LORA_BF16, 0), L.LORA_ESHAPE),
        (L.lora_relu2_mlp_desc(300, 256, 768, 16, 5, 0), L.LORA_EDTYPE),
    ]
    for desc, want in bad:
        assert _status(L, "lora_relu2_mlp_workspace_size", C.byref(desc), C.byref(f), C.byref(b)) == want
    d = L.lora_relu2_mlp_desc(128, 256, 768, 16, L.LORA_BF16, 0)
    _status(L, "lora_relu2_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    sv = L.lora_relu2_mlp_saved(FAKE, FAKE)
    up, dn = _proj(L), _proj(L)

    def fwd(X=FAKE, Y=FAKE * 2, saved=sv, ws=FAKE, nbytes=f.value):
        return _status(L, "lora_relu2_mlp_fwd", C.byref(d), X, C.byref(up), C.byref(dn), Y, C.byref(saved), ws,
                       nbytes, None)

    assert fwd(X=None) == L.LORA_EINVAL
    assert fwd(X=FAKE + 2) == L.LORA_EALIGN
    assert fwd(nbytes=f.value - 1) == L.LORA_EWORKSPACE
    assert fwd(saved=L.lora_relu2_mlp_saved(FAKE, None)) == L.LORA_EINVAL
    assert fwd(Y=FAKE) == L.LORA_EUNSUPPORTED  # Y aliases X


def test_plan_validation(L):
    """Per-call GEMM plans: value ranges, split-K only where a GEMM can split,
    unused entries zero; the workspace query sizes a forced split."""
    f, b = C.c_size_t(), C.c_size_t()

    def plan(g0=(0, 0), g1=(0, 0)):
        p = L.lora_plan()
        p.gemm[0].group, p.gemm[0].ksplit = g0
        p.gemm[1].group, p.gemm[1].ksplit = g1
        return p

    def mlp_ws(p):
        d = L.lora_mlp_desc(8192, 4096, 1024, 16, 0, L.LORA_BF16, C.pointer(p))
        st = _status(L, "lora_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b))
        return st, f.value, b.value

    st, f0, b0 = mlp_ws(plan())
    assert st == L.LORA_OK
    assert mlp_ws(plan(g0=(3, 0)))[0] == L.LORA_EINVAL        # group not a power of two
    assert mlp_ws(plan(g0=(64, 0)))[0] == L.LORA_EINVAL       # group too large
    assert mlp_ws(plan(g1=(8, 5)))[0] == L.LORA_EINVAL        # ksplit > 4
    assert mlp_ws(plan(g1=(8, -1)))[0] == L.LORA_EINVAL
    st, f4, b4 = mlp_ws(plan(g0=(16, 1), g1=(2, 4)))          # forced 4-way split of down and dX
    assert st == L.LORA_OK
    assert f4 - f0 >= 4 * 8192 * 4096 * 4 - 4096              # the down GEMM's fp32 parts
    assert b4 >= b0
    # the call rejects a split of an activation-epilogue GEMM before anything is enqueued
    sv = L.lora_mlp_saved(FAKE, FAKE, FAKE)
    g, u, dn = _proj(L), _proj(L), _proj(L)
    p = plan(g0=(4, 2))
    d = L.lora_mlp_desc(128, 256, 768, 16, 0, L.LORA_BF16, C.pointer(p))
    _status(L, "lora_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    st = _status(L, "lora_mlp_fwd", C.byref(d), FAKE, C.byref(g), C.byref(u), C.byref(dn), FAKE * 2, C.byref(sv),
                 FAKE * 3, f.value, None)
    assert st == L.LORA_EINVAL and b"only a dense plain-store GEMM" in L.load().lora_last_error()
    # an NF4 base cannot split either
    q = L.lora_nf4(FAKE, FAKE, FAKE, FAKE, 256, 768)
    p = plan(g0=(4, 2))
    do = L.lora_o_desc(64, 256, 768, 16, L.LORA_BF16, 0, C.pointer(p))
    _status(L, "lora_o_workspace_size", C.byref(do), C.byref(f), C.byref(b))
    st = _status(L, "lora_o_fwd", C.byref(do), FAKE, C.byref(_proj(L, W=None, nf4=q)), FAKE * 2, FAKE * 3, FAKE * 4,
                 f.value, None)
    assert st == L.LORA_EINVAL
    # a one-GEMM call takes no second entry; more parts than K steps are refused
    p = plan(g1=(4, 0))
    do = L.lora_o_desc(64, 256, 768, 16, L.LORA_BF16, 0, C.pointer(p))
    assert _status(L, "lora_o_workspace_size", C.byref(do), C.byref(f), C.byref(b)) == L.LORA_EINVAL
    p = plan(g0=(4, 4))
    do = L.lora_o_desc(64, 64, 768, 16, L.LORA_BF16, 0, C.pointer(p))  # K = 64 + the LoRA tile: 2 steps
    _status(L, "lora_o_workspace_size", C.byref(do), C.byref(f), C.byref(b))
    st = _status(L, "lora_o_fwd", C.byref(do), FAKE, C.byref(_proj(L)), FAKE * 2, FAKE * 3, FAKE * 4, f.value, None)
    assert st == L.LORA_EINVAL and b"exceeds the 2 K steps" in L.load().lora_last_error()


def test_plan_cache_round_trip(tmp_path, monkeypatch):
    """The tuner's JSON cache: entries are stored per device and shape, survive
    a reload, and a miss returns None (the library's defaults)."""
    from adapter_mlp_amd import tune

    monkeypatch.setattr(tune, "device_key", lambda device=None: "gfx950:256cu:test")
    path = str(tmp_path / "plans.json")
    c = tune.PlanCache(path)
    key = tune.mlp_key(3000, 2560, 9728, 16, "swiglu", 1, False)
    assert tune.cached(c, key) is None
    c.put(key, {"fwd": [[4, 0], [16, 2]], "bwd": [[2, 0], [8, 1]], "ms": {}})
    c2 = tune.PlanCache(path)
    assert tune.cached(c2, key) == {"fwd": [(4, 0), (16, 2)], "bwd": [(2, 0), (8, 1)]}
    monkeypatch.setattr(tune, "device_key", lambda device=None: "gfx942:304cu:other")
    assert tune.cached(c2, key) is None  # plans are per GPU


def test_validator_under_asan_ubsan(tmp_path):
    """The host code of csrc/abi.hip (validation, workspace planning, plans)
    built with AddressSanitizer and UndefinedBehaviorSanitizer, driven by
    tests/abi_sanitize_driver.cpp through failing calls and workspace
    queries only (no GPU needed); the other translation units are the
    regular build's objects.  Any sanitizer report aborts the driver."""
    import subprocess

    hipcc, clang = "/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang++"
    build = os.path.join(ROOT, "adapter_mlp_amd", "_build")
    others = [os.path.join(build, f + ".o") for f in ("gemm_bf16", "gemm_f32", "nf4", "skinny", "trace")]
    if not (os.path.exists(hipcc) and os.path.exists(clang) and all(map(os.path.exists, others))):
        pytest.skip("needs hipcc and the regular build's objects (python -m adapter_mlp_amd.build)")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "adapter_mlp_amd", "csrc")]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    abi_o, drv_o, exe = (str(tmp_path / n) for n in ("abi_san.o", "driver.o", "driver"))

    def run(cmd):
        p = subprocess.run(cmd, capture_output=True, text=True)
        assert p.returncode == 0, " ".join(cmd) + "\n" + p.stdout[-3000:] + p.stderr[-3000:]

    run([hipcc, "-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature",
         "-Xclang", "-packed-fp32-ops"] + san + inc +
        ["-c", os.path.join(ROOT, "adapter_mlp_amd", "csrc", "abi.hip"), "-o", abi_o])
    # the driver passes an out-of-range status on purpose (as a C caller may):
    # only its own enum loads go unchecked; the library's are checked
    run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize=enum",
         "-fno-sanitize-recover=undefined"] + inc +
        ["-c", os.path.join(ROOT, "tests", "abi_sanitize_driver.cpp"), "-o", drv_o])
    run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         drv_o, abi_o] + others + ["-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert p.returncode == 0, p.stdout[-3000:] + p.stderr[-3000:]
    assert "0 unexpected statuses" in p.stdout
