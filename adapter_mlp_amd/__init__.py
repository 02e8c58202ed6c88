"""Fused LoRA / QLoRA projections for AMD MI355X (gfx950).

Thin Python layer over the C-ABI library ``liblora_mi355x.so``: it allocates
outputs and workspace with PyTorch (device memory and streams only), fills
the C descriptors and calls the library.  All arithmetic runs in the
library's HIP kernels.

Layouts follow the C header: W [n_in, n_out], A [n_in, r], B [r, n_out],
row-major; bf16 or fp32 compute; NF4 bases in bf16.  bf16 inputs with fp32
adapters select the fp32 LoRA-gradient mode (fp32 dA, dB).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

from . import _lib as L

__all__ = [
    "Proj", "NF4Weight", "load", "LoraError",
    "mlp_fwd", "mlp_bwd", "mlp_workspace_size",
    "relu2_mlp_fwd", "relu2_mlp_bwd", "relu2_mlp_workspace_size",
    "qkv_fwd", "qkv_bwd", "o_fwd", "o_bwd", "o_fwd_noalloc",
    "nf4_quantize", "nf4_dequant", "nf4_unpack_codes", "nf4_gemm", "nf4_codebook",
    "trace_begin", "trace_end",
]

load = L.load
LoraError = L.LoraError


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return L.LORA_BF16
    if t.dtype == torch.float32:
        return L.LORA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _call_dtype(X, projs) -> int:
    """dtype code of a call: X's dtype, or the fp32 LoRA-gradient mode
    (LORA_BF16_F32LORA) when X is bf16 and the adapters are fp32.  Dense
    bases must have X's dtype."""
    torch = _torch()
    ad = {t.dtype for p in projs for t in (p.A, p.B)}
    if len(ad) != 1:
        raise ValueError(f"the adapters of one call must share a dtype, got {sorted(map(str, ad))}")
    for p in projs:
        if p.W is not None and p.W.dtype != X.dtype:
            raise ValueError(f"base weight dtype {p.W.dtype} differs from the input dtype {X.dtype}")
    (a,) = ad
    if a == X.dtype:
        return _dtype_code(X)
    if X.dtype == torch.bfloat16 and a == torch.float32:
        return L.LORA_BF16_F32LORA
    raise ValueError(f"adapters in {a} with inputs in {X.dtype} are not supported")


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _nbytes(ws, device) -> int:
    """Size in bytes of a caller's workspace tensor (dense, on the call's device)."""
    if not ws.is_contiguous():
        raise ValueError("ws is not contiguous")
    if ws.device != device:
        raise ValueError(f"ws is on {ws.device}, expected {device}")
    return ws.numel() * ws.element_size()


def _set_plan(desc, plan):
    """Put an optional GEMM launch plan into a call descriptor: a sequence of
    up to two (group, ksplit) pairs, the call's GEMMs in launch order (see
    lora_plan in the C header); None keeps the library's defaults.  The
    ctypes pointer keeps the struct alive as long as the descriptor."""
    if plan is None:
        return desc
    entries = list(plan)
    if len(entries) > 2:
        raise ValueError(f"a plan has at most two GEMM entries, got {len(entries)}")
    p = L.lora_plan()
    for i, e in enumerate(entries):
        g, k = (int(x) for x in e)
        p.gemm[i].group, p.gemm[i].ksplit = g, k
    desc.plan = C.pointer(p)
    return desc


def _on(stream):
    """Allocation context of a call: PyTorch's caching allocator ties every
    tensor allocated inside it (outputs, workspace) to the stream the library
    enqueues on, so a buffer is not handed to other work while the call's
    kernels may still use it."""
    import contextlib

    return contextlib.nullcontext() if stream is None else _torch().cuda.stream(stream)


def _need(name, t, shape, dtype, device):
    """Raise ValueError unless t is a dense tensor of this shape and dtype on
    this device (the kernels take row-major dense buffers)."""
    if t is None:
        raise ValueError(f"{name} is missing")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(int(x) for x in shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} is not contiguous (the library takes dense row-major buffers)")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (the device of X)")


def _on_gpu(X, ws=None):
    if ws is not None:
        _nbytes(ws, X.device)
    if X.device.type != "cuda":
        raise ValueError(f"X is on {X.device}: the library runs on the GPU only")


def _x2d(name, X):
    if X.dim() != 2:
        raise ValueError(f"{name} must be 2-D [tokens, width], got shape {tuple(X.shape)}")
    return X.shape


def _adapter_dtype(X, dt):
    torch = _torch()
    return torch.float32 if dt in (L.LORA_F32, L.LORA_BF16_F32LORA) else X.dtype


def _check_proj(name, p, n_in, n_out, r, X, dt):
    """A [n_in, r], B [r, n_out] in the call's adapter dtype; the base W
    [n_in, n_out] in X's dtype, or an NF4 weight of that shape."""
    torch = _torch()
    ad = _adapter_dtype(X, dt)
    _need(f"{name}.A", p.A, (n_in, r), ad, X.device)
    _need(f"{name}.B", p.B, (r, n_out), ad, X.device)
    if (p.W is None) == (p.nf4 is None):
        raise ValueError(f"{name}: exactly one of W and nf4 must be set")
    if p.Wt is not None:
        if p.W is None:
            raise ValueError(f"{name}: Wt is only for a dense W")
        _need(f"{name}.Wt", p.Wt, (n_out, n_in), X.dtype, X.device)
    if p.W is not None:
        _need(f"{name}.W", p.W, (n_in, n_out), X.dtype, X.device)
    else:
        w = p.nf4
        if (w.rows, w.cols) != (n_in, n_out):
            raise ValueError(f"{name}: NF4 weight is [{w.rows}, {w.cols}], expected [{n_in}, {n_out}]")
        _check_nf4(name, w, X.device)


def _check_nf4(name, w, device):
    torch = _torch()
    n = w.rows * w.cols
    if n % (64 * 256):
        raise ValueError(f"{name}: NF4 element count {n} is not a multiple of {64 * 256}")
    _need(f"{name}.codes", w.codes, (n // 2,), torch.uint8, device)
    _need(f"{name}.q8", w.q8, (n // 64,), torch.int8, device)
    _need(f"{name}.s2", w.s2, (n // (64 * 256),), torch.float32, device)
    _need(f"{name}.mu", w.mu, (1,), torch.float32, device)


@dataclass
class NF4Weight:
    """NF4-packed weight W [rows, cols] (device tensors)."""

    codes: object  # uint8 [numel/2]
    q8: object     # int8 [numel/64]
    s2: object     # float32 [numel/16384]
    mu: object     # float32 [1]
    rows: int
    cols: int

    def c_struct(self) -> L.lora_nf4:
        return L.lora_nf4(_ptr(self.codes), _ptr(self.q8), _ptr(self.s2), _ptr(self.mu), self.rows, self.cols)


@dataclass
class Proj:
    """One LoRA projection: dense W or NF4 weight, adapters A, B and scale s.
    Wt (optional, dense bf16 only): the same weight stored [n_out, n_in]
    (W.t().contiguous(), PyTorch nn.Linear's layout); the forward GEMMs read
    it when every projection they read has one."""

    A: object
    B: object
    scale: float
    W: object = None
    nf4: Optional[NF4Weight] = None
    Wt: object = None

    def c_struct(self, keep: list) -> L.lora_proj:
        p = L.lora_proj()
        p.W = _ptr(self.W)
        if self.nf4 is not None:
            s = self.nf4.c_struct()
            keep.append(s)
            p.nf4 = C.pointer(s)
        p.A = _ptr(self.A)
        p.B = _ptr(self.B)
        p.scale = float(self.scale)
        p.Wt = _ptr(self.Wt)
        return p


# ---------------------------------------------------------------------------
# MLP
# ---------------------------------------------------------------------------

def mlp_workspace_size(T, H, I, r, act="swiglu", dtype=L.LORA_BF16, plan=None):
    d = _set_plan(L.lora_mlp_desc(T, H, I, r, L.ACT_CODES[act], dtype), plan)
    f, b = C.c_size_t(), C.c_size_t()
    L.call("lora_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    return f.value, b.value


def _mlp_dims(X, gate, up, down):
    T, H = _x2d("X", X)
    if gate.A.dim() != 2 or gate.B.dim() != 2:
        raise ValueError("gate.A and gate.B must be 2-D")
    I, r = gate.B.shape[1], gate.A.shape[1]
    dt = _call_dtype(X, (gate, up, down))
    for name, p, n_in, n_out in (("gate", gate, H, I), ("up", up, H, I), ("down", down, I, H)):
        _check_proj(name, p, n_in, n_out, r, X, dt)
    return T, H, I, r, dt


def _check_saved(saved, names_shapes, X):
    if not isinstance(saved, dict):
        raise ValueError("saved must be the dict the forward returned")
    for k, shape in names_shapes:
        _need(f"saved[{k!r}]", saved.get(k), shape, X.dtype, X.device)


def mlp_fwd(X, gate: Proj, up: Proj, down: Proj, act="swiglu", *, Y=None, saved=None, ws=None, stream=None,
            plan=None):
    """Y = down(phi(gate(X)) * up(X)).  Returns (Y, saved) with saved = dict(e, g, U).

    Outputs and workspace the caller does not pass are allocated on ``stream``
    (default: the current stream), where the library enqueues its kernels."""
    torch = _torch()
    T, H, I, r, dt = _mlp_dims(X, gate, up, down)
    if act not in L.ACT_CODES:
        raise ValueError(f"unknown activation {act!r}")
    if Y is not None:
        _need("Y", Y, (T, H), X.dtype, X.device)
    if saved is not None:
        _check_saved(saved, (("e", (T, I)), ("g", (T, I)), ("U", (T, 3 * r))), X)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_mlp_desc(T, H, I, r, L.ACT_CODES[act], dt), plan)
    fb, _ = mlp_workspace_size(T, H, I, r, act, dt, plan)
    with _on(stream):
        if Y is None:
            Y = torch.empty((T, H), dtype=X.dtype, device=X.device)
        if saved is None:
            saved = dict(e=torch.empty((T, I), dtype=X.dtype, device=X.device),
                         g=torch.empty((T, I), dtype=X.dtype, device=X.device),
                         U=torch.empty((T, 3 * r), dtype=X.dtype, device=X.device))
        if ws is None:
            ws = _ws(fb, X.device)
    keep = []
    sv = L.lora_mlp_saved(_ptr(saved["e"]), _ptr(saved["g"]), _ptr(saved["U"]))
    L.call("lora_mlp_fwd", C.byref(d), _ptr(X), C.byref(gate.c_struct(keep)), C.byref(up.c_struct(keep)),
           C.byref(down.c_struct(keep)), _ptr(Y), C.byref(sv), _ptr(ws), _nbytes(ws, X.device), _stream(stream))
    return Y, saved


_MLP_GRAD_KEYS = ("dA_gate", "dB_gate", "dA_up", "dB_up", "dA_down", "dB_down")


def mlp_bwd(dY, X, saved, gate: Proj, up: Proj, down: Proj, act="swiglu", *, dX=None, grads=None, ws=None,
            stream=None, plan=None):
    """Returns (dX, grads) with grads = dict(dA_gate, dB_gate, dA_up, dB_up, dA_down, dB_down).
    ``dX=X`` writes the input gradient over X."""
    torch = _torch()
    T, H, I, r, dt = _mlp_dims(X, gate, up, down)
    if act not in L.ACT_CODES:
        raise ValueError(f"unknown activation {act!r}")
    _need("dY", dY, (T, H), X.dtype, X.device)
    _check_saved(saved, (("e", (T, I)), ("g", (T, I)), ("U", (T, 3 * r))), X)
    if dX is not None:
        _need("dX", dX, (T, H), X.dtype, X.device)
    if grads is not None:
        for k, p, ab in zip(_MLP_GRAD_KEYS, (gate, gate, up, up, down, down), "ABABAB"):
            ref = getattr(p, ab)
            _need(f"grads[{k!r}]", grads.get(k), ref.shape, ref.dtype, X.device)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_mlp_desc(T, H, I, r, L.ACT_CODES[act], dt), plan)
    _, bb = mlp_workspace_size(T, H, I, r, act, dt, plan)
    with _on(stream):
        if dX is None:
            dX = torch.empty_like(X)
        if grads is None:
            grads = dict(dA_gate=torch.empty_like(gate.A), dB_gate=torch.empty_like(gate.B),
                         dA_up=torch.empty_like(up.A), dB_up=torch.empty_like(up.B),
                         dA_down=torch.empty_like(down.A), dB_down=torch.empty_like(down.B))
        if ws is None:
            ws = _ws(bb, X.device)
    keep = []
    sv = L.lora_mlp_saved(_ptr(saved["e"]), _ptr(saved["g"]), _ptr(saved["U"]))
    gr = L.lora_mlp_grads(*(_ptr(grads[k]) for k in _MLP_GRAD_KEYS))
    L.call("lora_mlp_bwd", C.byref(d), _ptr(dY), _ptr(X), C.byref(sv), C.byref(gate.c_struct(keep)),
           C.byref(up.c_struct(keep)), C.byref(down.c_struct(keep)), _ptr(dX), C.byref(gr), _ptr(ws),
           _nbytes(ws, X.device), _stream(stream))
    return dX, grads


# ---------------------------------------------------------------------------
# Ungated ReLU^2 MLP
# ---------------------------------------------------------------------------

def relu2_mlp_workspace_size(T, H, I, r, dtype=L.LORA_BF16, plan=None):
    d = _set_plan(L.lora_relu2_mlp_desc(T, H, I, r, dtype, 0), plan)
    f, b = C.c_size_t(), C.c_size_t()
    L.call("lora_relu2_mlp_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    return f.value, b.value


def _relu2_dims(X, up, down):
    T, H = _x2d("X", X)
    if up.A.dim() != 2 or up.B.dim() != 2:
        raise ValueError("up.A and up.B must be 2-D")
    I, r = up.B.shape[1], up.A.shape[1]
    dt = _call_dtype(X, (up, down))
    _check_proj("up", up, H, I, r, X, dt)
    _check_proj("down", down, I, H, r, X, dt)
    return T, H, I, r, dt


def relu2_mlp_fwd(X, up: Proj, down: Proj, *, Y=None, saved=None, ws=None, stream=None, plan=None):
    """Y = down(relu(up(X))^2).  Returns (Y, saved) with saved = dict(u, U)."""
    torch = _torch()
    T, H, I, r, dt = _relu2_dims(X, up, down)
    if Y is not None:
        _need("Y", Y, (T, H), X.dtype, X.device)
    if saved is not None:
        _check_saved(saved, (("u", (T, I)), ("U", (T, 2 * r))), X)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_relu2_mlp_desc(T, H, I, r, dt, 0), plan)
    fb, _ = relu2_mlp_workspace_size(T, H, I, r, dt, plan)
    with _on(stream):
        if Y is None:
            Y = torch.empty((T, H), dtype=X.dtype, device=X.device)
        if saved is None:
            saved = dict(u=torch.empty((T, I), dtype=X.dtype, device=X.device),
                         U=torch.empty((T, 2 * r), dtype=X.dtype, device=X.device))
        if ws is None:
            ws = _ws(fb, X.device)
    keep = []
    sv = L.lora_relu2_mlp_saved(_ptr(saved["u"]), _ptr(saved["U"]))
    L.call("lora_relu2_mlp_fwd", C.byref(d), _ptr(X), C.byref(up.c_struct(keep)), C.byref(down.c_struct(keep)),
           _ptr(Y), C.byref(sv), _ptr(ws), _nbytes(ws, X.device), _stream(stream))
    return Y, saved


_RELU2_GRAD_KEYS = ("dA_up", "dB_up", "dA_down", "dB_down")


def relu2_mlp_bwd(dY, X, saved, up: Proj, down: Proj, *, dX=None, grads=None, ws=None, stream=None, plan=None):
    """Returns (dX, grads) with grads = dict(dA_up, dB_up, dA_down, dB_down)."""
    torch = _torch()
    T, H, I, r, dt = _relu2_dims(X, up, down)
    _need("dY", dY, (T, H), X.dtype, X.device)
    _check_saved(saved, (("u", (T, I)), ("U", (T, 2 * r))), X)
    if dX is not None:
        _need("dX", dX, (T, H), X.dtype, X.device)
    if grads is not None:
        for k, p, ab in zip(_RELU2_GRAD_KEYS, (up, up, down, down), "ABAB"):
            ref = getattr(p, ab)
            _need(f"grads[{k!r}]", grads.get(k), ref.shape, ref.dtype, X.device)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_relu2_mlp_desc(T, H, I, r, dt, 0), plan)
    _, bb = relu2_mlp_workspace_size(T, H, I, r, dt, plan)
    with _on(stream):
        if dX is None:
            dX = torch.empty_like(X)
        if grads is None:
            grads = dict(dA_up=torch.empty_like(up.A), dB_up=torch.empty_like(up.B),
                         dA_down=torch.empty_like(down.A), dB_down=torch.empty_like(down.B))
        if ws is None:
            ws = _ws(bb, X.device)
    keep = []
    sv = L.lora_relu2_mlp_saved(_ptr(saved["u"]), _ptr(saved["U"]))
    gr = L.lora_relu2_mlp_grads(*(_ptr(grads[k]) for k in _RELU2_GRAD_KEYS))
    L.call("lora_relu2_mlp_bwd", C.byref(d), _ptr(dY), _ptr(X), C.byref(sv), C.byref(up.c_struct(keep)),
           C.byref(down.c_struct(keep)), _ptr(dX), C.byref(gr), _ptr(ws), _nbytes(ws, X.device), _stream(stream))
    return dX, grads


# ---------------------------------------------------------------------------
# Q/K/V and O
# ---------------------------------------------------------------------------

def qkv_workspace_size(T, H, Nq, Nk, Nv, r, dtype=L.LORA_BF16, plan=None):
    d = _set_plan(L.lora_qkv_desc(T, H, Nq, Nk, Nv, r, dtype, 0), plan)
    f, b = C.c_size_t(), C.c_size_t()
    L.call("lora_qkv_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    return f.value, b.value


def _qkv_dims(X, q, k, v):
    T, H = _x2d("X", X)
    if q.A.dim() != 2 or any(p.B.dim() != 2 for p in (q, k, v)):
        raise ValueError("adapters must be 2-D")
    Ns = [p.B.shape[1] for p in (q, k, v)]
    r = q.A.shape[1]
    dt = _call_dtype(X, (q, k, v))
    for name, p, n in zip("qkv", (q, k, v), Ns):
        _check_proj(name, p, H, n, r, X, dt)
    return T, H, Ns, r, dt


_QKV_GRAD_KEYS = ("dA_q", "dB_q", "dA_k", "dB_k", "dA_v", "dB_v")


def qkv_fwd(X, q: Proj, k: Proj, v: Proj, *, out=None, U=None, ws=None, stream=None, plan=None):
    """Returns (Q, K, V, U) with U = [X A_q | X A_k | X A_v]."""
    torch = _torch()
    T, H, Ns, r, dt = _qkv_dims(X, q, k, v)
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must hold three tensors (Q, K, V)")
        for name, t, n in zip("QKV", out, Ns):
            _need(name, t, (T, n), X.dtype, X.device)
    if U is not None:
        _need("U", U, (T, 3 * r), X.dtype, X.device)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_qkv_desc(T, H, Ns[0], Ns[1], Ns[2], r, dt, 0), plan)
    fb, _ = qkv_workspace_size(T, H, *Ns, r, dt, plan)
    with _on(stream):
        if out is None:
            out = [torch.empty((T, n), dtype=X.dtype, device=X.device) for n in Ns]
        if U is None:
            U = torch.empty((T, 3 * r), dtype=X.dtype, device=X.device)
        if ws is None:
            ws = _ws(fb, X.device)
    keep = []
    L.call("lora_qkv_fwd", C.byref(d), _ptr(X), C.byref(q.c_struct(keep)), C.byref(k.c_struct(keep)),
           C.byref(v.c_struct(keep)), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(U), _ptr(ws), _nbytes(ws, X.device),
           _stream(stream))
    return out[0], out[1], out[2], U


def qkv_bwd(dQ, dK, dV, X, U, q: Proj, k: Proj, v: Proj, *, dX=None, grads=None, ws=None, stream=None,
            plan=None):
    """Returns (dX, grads) with grads = dict(dA_q, dB_q, dA_k, dB_k, dA_v, dB_v).
    ``dX=X`` writes the input gradient over X."""
    torch = _torch()
    T, H, Ns, r, dt = _qkv_dims(X, q, k, v)
    for name, t, n in (("dQ", dQ, Ns[0]), ("dK", dK, Ns[1]), ("dV", dV, Ns[2])):
        _need(name, t, (T, n), X.dtype, X.device)
    _need("U", U, (T, 3 * r), X.dtype, X.device)
    if dX is not None:
        _need("dX", dX, (T, H), X.dtype, X.device)
    if grads is not None:
        for key, p, ab in zip(_QKV_GRAD_KEYS, (q, q, k, k, v, v), "ABABAB"):
            ref = getattr(p, ab)
            _need(f"grads[{key!r}]", grads.get(key), ref.shape, ref.dtype, X.device)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_qkv_desc(T, H, Ns[0], Ns[1], Ns[2], r, dt, 0), plan)
    _, bb = qkv_workspace_size(T, H, *Ns, r, dt, plan)
    with _on(stream):
        if dX is None:
            dX = torch.empty_like(X)
        if grads is None:
            grads = dict(dA_q=torch.empty_like(q.A), dB_q=torch.empty_like(q.B), dA_k=torch.empty_like(k.A),
                         dB_k=torch.empty_like(k.B), dA_v=torch.empty_like(v.A), dB_v=torch.empty_like(v.B))
        if ws is None:
            ws = _ws(bb, X.device)
    keep = []
    gr = L.lora_qkv_grads(*(_ptr(grads[n]) for n in _QKV_GRAD_KEYS))
    L.call("lora_qkv_bwd", C.byref(d), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(X), _ptr(U), C.byref(q.c_struct(keep)),
           C.byref(k.c_struct(keep)), C.byref(v.c_struct(keep)), _ptr(dX), C.byref(gr), _ptr(ws), _nbytes(ws, X.device),
           _stream(stream))
    return dX, grads


def o_workspace_size(T, K, N, r, dtype=L.LORA_BF16, plan=None):
    d = _set_plan(L.lora_o_desc(T, K, N, r, dtype, 0), plan)
    f, b = C.c_size_t(), C.c_size_t()
    L.call("lora_o_workspace_size", C.byref(d), C.byref(f), C.byref(b))
    return f.value, b.value


def _o_dims(X, o):
    T, K = _x2d("X", X)
    if o.A.dim() != 2 or o.B.dim() != 2:
        raise ValueError("o.A and o.B must be 2-D")
    N, r = o.B.shape[1], o.A.shape[1]
    dt = _call_dtype(X, (o,))
    _check_proj("o", o, K, N, r, X, dt)
    return T, K, N, r, dt


def o_fwd(X, o: Proj, *, Y=None, U=None, ws=None, stream=None, plan=None):
    """Returns (Y, U)."""
    torch = _torch()
    T, K, N, r, dt = _o_dims(X, o)
    if Y is not None:
        _need("Y", Y, (T, N), X.dtype, X.device)
    if U is not None:
        _need("U", U, (T, r), X.dtype, X.device)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_o_desc(T, K, N, r, dt, 0), plan)
    fb, _ = o_workspace_size(T, K, N, r, dt, plan)
    with _on(stream):
        if Y is None:
            Y = torch.empty((T, N), dtype=X.dtype, device=X.device)
        if U is None:
            U = torch.empty((T, r), dtype=X.dtype, device=X.device)
        if ws is None:
            ws = _ws(fb, X.device)
    keep = []
    L.call("lora_o_fwd", C.byref(d), _ptr(X), C.byref(o.c_struct(keep)), _ptr(Y), _ptr(U), _ptr(ws), _nbytes(ws, X.device),
           _stream(stream))
    return Y, U


def o_fwd_noalloc(X, o: Proj, *, Y, U, stream=None, plan=None):
    """o_fwd for callers that cannot allocate: the library takes its scratch
    from a static per-GPU array (at most NOALLOC_SCRATCH_BYTES, shared by all
    such calls on that GPU) and allocates nothing; the caller passes the
    outputs Y [T, N] and U [T, r].  Returns (Y, U)."""
    T, K, N, r, dt = _o_dims(X, o)
    _need("Y", Y, (T, N), X.dtype, X.device)
    _need("U", U, (T, r), X.dtype, X.device)
    _on_gpu(X)
    d = _set_plan(L.lora_o_desc(T, K, N, r, dt, 0), plan)
    keep = []
    L.call("lora_o_fwd_noalloc", C.byref(d), _ptr(X), C.byref(o.c_struct(keep)), _ptr(Y), _ptr(U),
           _stream(stream))
    return Y, U


NOALLOC_SCRATCH_BYTES = L.NOALLOC_SCRATCH_BYTES


def o_bwd(dY, X, U, o: Proj, *, dX=None, dA=None, dB=None, ws=None, stream=None, plan=None):
    """Returns (dX, dA, dB).  ``dX=X`` writes the input gradient over X."""
    torch = _torch()
    T, K, N, r, dt = _o_dims(X, o)
    _need("dY", dY, (T, N), X.dtype, X.device)
    _need("U", U, (T, r), X.dtype, X.device)
    if dX is not None:
        _need("dX", dX, (T, K), X.dtype, X.device)
    if dA is not None:
        _need("dA", dA, o.A.shape, o.A.dtype, X.device)
    if dB is not None:
        _need("dB", dB, o.B.shape, o.B.dtype, X.device)
    _on_gpu(X, ws)
    d = _set_plan(L.lora_o_desc(T, K, N, r, dt, 0), plan)
    _, bb = o_workspace_size(T, K, N, r, dt, plan)
    with _on(stream):
        dX = torch.empty_like(X) if dX is None else dX
        dA = torch.empty_like(o.A) if dA is None else dA
        dB = torch.empty_like(o.B) if dB is None else dB
        if ws is None:
            ws = _ws(bb, X.device)
    keep = []
    L.call("lora_o_bwd", C.byref(d), _ptr(dY), _ptr(X), _ptr(U), C.byref(o.c_struct(keep)), _ptr(dX), _ptr(dA),
           _ptr(dB), _ptr(ws), _nbytes(ws, X.device), _stream(stream))
    return dX, dA, dB


# ---------------------------------------------------------------------------
# NF4
# ---------------------------------------------------------------------------

def nf4_codebook():
    buf = (C.c_float * 16)()
    L.load().lora_nf4_codebook(buf)
    return list(buf)


def nf4_quantize(W, *, stream=None) -> NF4Weight:
    """Quantize a device weight W [rows, cols] (fp32 or bf16) to NF4 on the GPU."""
    torch = _torch()
    rows, cols = _x2d("W", W)
    if not W.is_contiguous():
        raise ValueError("W is not contiguous (the library takes dense row-major buffers)")
    _dtype_code(W)
    _on_gpu(W)
    n = rows * cols
    nbytes = C.c_size_t()
    L.call("lora_nf4_quantize_workspace_size", rows, cols, C.byref(nbytes))
    dev = W.device
    with _on(stream):
        w = NF4Weight(codes=torch.empty(n // 2, dtype=torch.uint8, device=dev),
                      q8=torch.empty(n // 64, dtype=torch.int8, device=dev),
                      s2=torch.empty(n // 16384, dtype=torch.float32, device=dev),
                      mu=torch.empty(1, dtype=torch.float32, device=dev), rows=rows, cols=cols)
        ws = _ws(nbytes.value, dev)
    L.call("lora_nf4_quantize", _ptr(W), rows, cols, _dtype_code(W), _ptr(w.codes), _ptr(w.q8), _ptr(w.s2),
           _ptr(w.mu), _ptr(ws), _nbytes(ws, dev), _stream(stream))
    return w


def nf4_dequant(w: NF4Weight, dtype=None, *, out=None, stream=None):
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    _check_nf4("w", w, w.codes.device)
    if out is not None:
        _need("out", out, (w.rows, w.cols), dtype, w.codes.device)
    _on_gpu(w.codes)
    with _on(stream):
        if out is None:
            out = torch.empty((w.rows, w.cols), dtype=dtype, device=w.codes.device)
    s = w.c_struct()
    L.call("lora_nf4_dequant", C.byref(s), _ptr(out), _dtype_code(out), _stream(stream))
    return out


def nf4_unpack_codes(w: NF4Weight, *, stream=None):
    torch = _torch()
    _check_nf4("w", w, w.codes.device)
    _on_gpu(w.codes)
    with _on(stream):
        out = torch.empty(w.rows * w.cols, dtype=torch.uint8, device=w.codes.device)
    s = w.c_struct()
    L.call("lora_nf4_unpack_codes", C.byref(s), _ptr(out), _stream(stream))
    return out


def nf4_gemm(X, w: NF4Weight, A=None, B=None, scale=0.0, trans=False, *, Y=None, ws=None, stream=None):
    """trans=False: Y = X deq(W) + s (X A) B;  trans=True: Y = X deq(W)^T + s (X B^T) A^T."""
    torch = _torch()
    T, width = _x2d("X", X)
    k_in, n_out = (w.cols, w.rows) if trans else (w.rows, w.cols)
    if X.dtype != torch.bfloat16:
        raise ValueError(f"X has dtype {X.dtype}; the NF4 GEMM computes in bf16")
    _need("X", X, (T, k_in), torch.bfloat16, X.device)
    _check_nf4("w", w, X.device)
    if (A is None) != (B is None):
        raise ValueError("A and B must both be given or both be None")
    r = 0 if A is None else A.shape[1]
    if A is not None:
        _need("A", A, (w.rows, r), torch.bfloat16, X.device)
        _need("B", B, (r, w.cols), torch.bfloat16, X.device)
    if Y is not None:
        _need("Y", Y, (T, n_out), torch.bfloat16, X.device)
    _on_gpu(X, ws)
    nbytes = C.c_size_t()
    L.call("lora_nf4_gemm_workspace_size", T, w.rows, w.cols, r, int(trans), C.byref(nbytes))
    with _on(stream):
        if Y is None:
            Y = torch.empty((T, n_out), dtype=X.dtype, device=X.device)
        if ws is None:
            ws = _ws(nbytes.value, X.device)
    s = w.c_struct()
    L.call("lora_nf4_gemm", T, int(trans), _ptr(X), C.byref(s), _ptr(A), _ptr(B), r, float(scale), _ptr(Y),
           _ptr(ws), _nbytes(ws, X.device), _stream(stream))
    return Y


# ---------------------------------------------------------------------------
# Kernel timing
# ---------------------------------------------------------------------------

def trace_begin(prefix: str = "") -> None:
    """Record HIP-event durations of the library's launches (optionally only
    kernel families whose name starts with ``prefix``)."""
    L.call("lora_trace_begin", prefix.encode() if prefix else None)


def trace_end() -> dict:
    """Stop recording; returns {family: (launches, total_ms)}."""
    buf = (L.lora_trace_entry * 64)()
    n = C.c_int32()
    L.call("lora_trace_end", buf, 64, C.byref(n))
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n.value, 64))}
