"""Oracle for the LoRA projection, the gated LoRA MLP block and the LoRA
Q/K/V and O projections -- forward and analytic backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Layout (row-major throughout): a projection maps width ``n_in`` to ``n_out``
with a frozen base ``W [n_in, n_out]``, adapters ``A [n_in, r]`` and
``B [r, n_out]`` and a scalar ``s`` (alpha / r).  Inside the pages' autograd
functions the adapters appear exactly this way round (``dY @ B.t()`` needs
``B [r, out]``, ``A.t() @ X.t()`` needs ``A [in, r]``); their base weight is
an ``nn.Linear`` ``[out, in]`` used as ``X @ W.t()``, which is the same
product as ``X @ W`` with ``W`` stored ``[in, out]``.

Every function works in the dtype of its inputs (float32 for parity, float64
for the pins) and uses nothing but numpy array expressions and ``@``.

Parity pins (tests/test_oracle_lora.py): central finite differences in
float64 for every gradient (gated and ReLU^2 MLPs, QKV, O), the merged-weight
closed form ``W + s*A@B``,
B = 0 / A = 0 / s = 0 special cases, hoisted-vs-recomputed bitwise identity,
token permutation, QKV = three single projections, activation special values
and the exact-GELU bound.
"""
from __future__ import annotations

import numpy as np

from .nf4 import round_to_bf16

# --------------------------------------------------------------------------
# Activations.  "LoRA Optimizations", section "Triton kernels": the MLP uses a
# SwiGLU or a GeGLU activation with fused forward and backward kernels; the
# backward returns the activation output together with both input gradients
# (section "Integration").  SiLU with beta = 1; GELU in its tanh form
# (Hendrycks & Gimpel), which the Gemma-style workload fixes.
# --------------------------------------------------------------------------

_SQRT_2_OVER_PI = 0.7978845608028654  # sqrt(2 / pi)
_GELU_C = 0.044715


def sigmoid(x):
    one = np.asarray(1, dtype=x.dtype)
    with np.errstate(over="ignore"):  # exp(-x) -> inf gives sigmoid 0, as it should
        return one / (one + np.exp(-x))


def silu(x):
    """phi(x) = x * sigmoid(x)."""
    return x * sigmoid(x)


def silu_grad(x):
    """phi'(x) = sigmoid(x) * (1 + x * (1 - sigmoid(x)))."""
    sg = sigmoid(x)
    return sg * (1 + x * (1 - sg))


def gelu_tanh(x):
    """phi(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))."""
    c = np.asarray(_SQRT_2_OVER_PI, dtype=x.dtype)
    k = np.asarray(_GELU_C, dtype=x.dtype)
    u = c * (x + k * x * x * x)
    return 0.5 * x * (1 + np.tanh(u))


def gelu_tanh_grad(x):
    """phi'(x) = (1 + tanh u)/2 + x/2 * (1 - tanh(u)^2) * sqrt(2/pi) * (1 + 3*0.044715 x^2)."""
    c = np.asarray(_SQRT_2_OVER_PI, dtype=x.dtype)
    k = np.asarray(_GELU_C, dtype=x.dtype)
    u = c * (x + k * x * x * x)
    t = np.tanh(u)
    return 0.5 * (1 + t) + 0.5 * x * (1 - t * t) * c * (1 + 3 * k * x * x)


ACTIVATIONS = {
    "swiglu": (silu, silu_grad),
    "geglu_tanh": (gelu_tanh, gelu_tanh_grad),
}


# --------------------------------------------------------------------------
# One LoRA projection ("LoRA_W" in the unsloth diff; the projection helper
# ``matmul_lora``).  The diff prints the base branch of ``matmul_lora`` only;
# the adapter term is the one whose gradients the backward hunks compute:
#     U = X @ A,   Z = X @ W + s * (U @ B)        (associated as written)
# --------------------------------------------------------------------------


def proj_fwd(X, W, A, B, s):
    """Forward of one LoRA projection.  Returns (Z, U) with U = X @ A saved."""
    U = X @ A
    Z = X @ W + s * (U @ B)
    return Z, U


def proj_bwd(dZ, X, W, A, B, s, U, hoist=True):
    """Backward of one LoRA projection (unsloth diff, ``LoRA_W.backward``).

    With ``P = dZ @ B.T`` (the "LoRA-B projected gradient", shape [T, r]):
        dA = s * X.T @ P
        dB = s * U.T @ dZ        (U = X @ A; the page forms it as A.t() @ X.t())
        dX = dZ @ W.T + s * P @ A.T
    The commit message of the diff hoists ``P`` so it is formed once and used
    for both dA and dX; ``hoist=False`` forms it separately for each use, as
    before that commit (the two must agree bit for bit).
    """
    P_for_dA = dZ @ B.T
    P_for_dX = P_for_dA if hoist else dZ @ B.T
    dA = s * (X.T @ P_for_dA)
    dB = s * (U.T @ dZ)
    dX = dZ @ W.T + s * (P_for_dX @ A.T)
    return dX, dA, dB


# --------------------------------------------------------------------------
# LoRA MLP block (unsloth diff, ``LoRA_MLP``; "LoRA Optimizations", section
# "Custom autograd functions").  e = gate projection, g = up projection,
# h = phi(e) * g, Y = down projection of h.  The gate side is the activated
# one: the diff pairs ``de`` with ``gateB`` and ``df`` with ``upB``.
# --------------------------------------------------------------------------


def mlp_fwd(X, gate, up, down, act="swiglu"):
    """Forward.  ``gate``/``up``/``down`` are dicts with W, A, B, s.

    Returns (Y, saved) where saved = dict(e, g, U_g, U_u, U_d)."""
    phi, _ = ACTIVATIONS[act]
    e, U_g = proj_fwd(X, gate["W"], gate["A"], gate["B"], gate["s"])
    g, U_u = proj_fwd(X, up["W"], up["A"], up["B"], up["s"])
    h = phi(e) * g
    Y, U_d = proj_fwd(h, down["W"], down["A"], down["B"], down["s"])
    return Y, dict(e=e, g=g, U_g=U_g, U_u=U_u, U_d=U_d)


def mlp_bwd(dY, X, saved, gate, up, down, act="swiglu", hoist=True):
    """Backward of the LoRA MLP block, given the upstream gradient dY.

    The page's hunks show the adapter gradients of down, up and gate, the
    hoisted ``df @ upB.t()`` / ``de @ gateB.t()`` products and the dX chain;
    the step between (dh = gradient of the down projection's input, then the
    activation backward that returns h, df, de) lies outside the printed
    hunks and follows from the forward:
        dh  = dY @ W_d.T + s_d * (dY @ B_d.T) @ A_d.T
        dg  = dh * phi(e)               (the page's ``df``)
        de  = dh * g * phi'(e)
        dX  = dg @ W_u.T + s_u*(dg @ B_u.T) @ A_u.T + de @ W_g.T + s_g*(de @ B_g.T) @ A_g.T
    Returns dict(dX, dA_g, dB_g, dA_u, dB_u, dA_d, dB_d).
    """
    phi, dphi = ACTIVATIONS[act]
    e, g = saved["e"], saved["g"]
    h = phi(e) * g
    dh, dA_d, dB_d = proj_bwd(dY, h, down["W"], down["A"], down["B"], down["s"], saved["U_d"], hoist)
    dg = dh * phi(e)
    de = dh * g * dphi(e)
    dX_u, dA_u, dB_u = proj_bwd(dg, X, up["W"], up["A"], up["B"], up["s"], saved["U_u"], hoist)
    dX_g, dA_g, dB_g = proj_bwd(de, X, gate["W"], gate["A"], gate["B"], gate["s"], saved["U_g"], hoist)
    dX = dX_u + dX_g
    return dict(dX=dX, dA_g=dA_g, dB_g=dB_g, dA_u=dA_u, dB_u=dB_u, dA_d=dA_d, dB_d=dB_d)


# --------------------------------------------------------------------------
# Ungated ReLU^2 MLP ("LoRA Optimizations", section "FP32 LoRA gradients":
# the dense ReLU^2 MLPs of Nemotron-H run up and down LoRA projections with a
# fused ReLU^2 activation derivative).  u = up projection, h = max(u, 0)^2,
# Y = down projection of h; there is no gate.
# --------------------------------------------------------------------------


def relu2(x):
    r = np.maximum(x, 0)
    return r * r


def relu2_grad(x):
    return 2 * np.maximum(x, 0)


def relu2_mlp_fwd(X, up, down):
    """Forward.  Returns (Y, saved) with saved = dict(u, U_u, U_d)."""
    u, U_u = proj_fwd(X, up["W"], up["A"], up["B"], up["s"])
    h = relu2(u)
    Y, U_d = proj_fwd(h, down["W"], down["A"], down["B"], down["s"])
    return Y, dict(u=u, U_u=U_u, U_d=U_d)


def relu2_mlp_bwd(dY, X, saved, up, down, hoist=True):
    """Backward: the down projection's gradients at h = relu2(u) give dh, the
    activation derivative gives du = dh * 2 max(u, 0), and the up
    projection's gradients at X follow.  Returns dict(dX, dA_u, dB_u, dA_d,
    dB_d)."""
    u = saved["u"]
    h = relu2(u)
    dh, dA_d, dB_d = proj_bwd(dY, h, down["W"], down["A"], down["B"], down["s"], saved["U_d"], hoist)
    du = dh * relu2_grad(u)
    dX, dA_u, dB_u = proj_bwd(du, X, up["W"], up["A"], up["B"], up["s"], saved["U_u"], hoist)
    return dict(dX=dX, dA_u=dA_u, dB_u=dB_u, dA_d=dA_d, dB_d=dB_d)


# --------------------------------------------------------------------------
# LoRA Q/K/V (unsloth diff, ``LoRA_QKV``): three projections of one X; the
# input gradient is the sum of the three projections' input gradients, each
# with its own hoisted dZ @ B.t().  O is a single projection (``LoRA_W``,
# ``apply_lora_o``).
# --------------------------------------------------------------------------


def qkv_fwd(X, q, k, v):
    Q, U_q = proj_fwd(X, q["W"], q["A"], q["B"], q["s"])
    K, U_k = proj_fwd(X, k["W"], k["A"], k["B"], k["s"])
    V, U_v = proj_fwd(X, v["W"], v["A"], v["B"], v["s"])
    return (Q, K, V), dict(U_q=U_q, U_k=U_k, U_v=U_v)


def qkv_bwd(dQ, dK, dV, X, saved, q, k, v, hoist=True):
    dX_q, dA_q, dB_q = proj_bwd(dQ, X, q["W"], q["A"], q["B"], q["s"], saved["U_q"], hoist)
    dX_k, dA_k, dB_k = proj_bwd(dK, X, k["W"], k["A"], k["B"], k["s"], saved["U_k"], hoist)
    dX_v, dA_v, dB_v = proj_bwd(dV, X, v["W"], v["A"], v["B"], v["s"], saved["U_v"], hoist)
    dX = dX_q + dX_k + dX_v
    return dict(dX=dX, dA_q=dA_q, dB_q=dB_q, dA_k=dA_k, dB_k=dB_k, dA_v=dA_v, dB_v=dB_v)


def o_fwd(X, o):
    Y, U = proj_fwd(X, o["W"], o["A"], o["B"], o["s"])
    return Y, dict(U=U)


def o_bwd(dY, X, saved, o, hoist=True):
    dX, dA, dB = proj_bwd(dY, X, o["W"], o["A"], o["B"], o["s"], saved["U"], hoist)
    return dict(dX=dX, dA=dA, dB=dB)


# --------------------------------------------------------------------------
# fp32 LoRA-gradient mode ("LoRA Optimizations", section "FP32 LoRA
# gradients"): the adapters and their gradients are fp32 while the products
# keep 16-bit inputs, and the parameter gradients come out in fp32.  The
# unsloth diff's backward casts every adapter to the compute dtype before its
# first product (``gateA.to(dtype)`` and so on in LoRA_MLP and LoRA_QKV), so
# the mode multiplies with the adapters rounded to bf16.
# --------------------------------------------------------------------------


def to_compute_adapters(p):
    """Projection dict with A and B rounded to bf16 (nearest even), held in
    fp32: the adapters the fp32 LoRA-gradient mode multiplies with.  Given
    these, the functions above produce that mode's outputs; its dA and dB are
    their fp32 gradients as they stand, with no rounding to bf16."""
    q = dict(p)
    q["A"] = round_to_bf16(np.asarray(p["A"], dtype=np.float32))
    q["B"] = round_to_bf16(np.asarray(p["B"], dtype=np.float32))
    return q


def as_dtype(p, dtype):
    """Copy of a projection dict (W, A, B, s) with arrays cast to ``dtype``."""
    return {kk: (np.asarray(vv, dtype=dtype) if kk != "s" else vv) for kk, vv in p.items()}
