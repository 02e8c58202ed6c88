"""Seeded input generation (shapes, distributions, seeds).

Distributions follow the workload descriptions of the five benchmark shapes:

* base weights ``W ~ N(0, 1/fan_in)`` (standard deviation ``1/sqrt(fan_in)``),
  stored ``[in, out]`` row-major;
* adapter ``A ~ U(-1/sqrt(fan_in), 1/sqrt(fan_in))`` (the Kaiming-uniform
  bound of a linear layer), stored ``[in, r]``;
* adapter ``B ~ N(0, 0.02)`` (non-zero, so every gradient is exercised),
  stored ``[r, out]``;
* activations ``X`` and upstream gradients ``dY ~ N(0, 1)``; where the shape
  stands for an RMSNorm output, each row is divided by
  ``sqrt(mean(x^2) + 1e-6)`` (gain 1).

For 16-bit configurations every tensor is rounded to bfloat16
(round-to-nearest-even) here, once, and handed out as float32 arrays that hold
bf16-representable values, so that the oracle and the GPU path consume
identical numbers.  The one exception is ``lora_dtype="f32"`` (the fp32
LoRA-gradient mode): there the adapters ``A`` and ``B`` stay full fp32 values.

Every tensor has its own stream: ``numpy.random.default_rng([seed, fnv1a(name)])``
with ``seed = 1000 + config id`` unless a caller passes another seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


def fnv1a32(name: str) -> int:
    """32-bit FNV-1a hash of a tensor name (substream key)."""
    h = 0x811C9DC5
    for b in name.encode():
        h ^= b
        h = (h * 0x01000193) & 0xFFFFFFFF
    return h


def rng_for(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), fnv1a32(name)])


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even);
    returns float32.  In place on a private copy, uint32 arithmetic (no
    overflow for finite inputs)."""
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


@dataclass(frozen=True)
class WorkloadConfig:
    """One benchmark shape.  ``kind`` is ``"mlp"`` (gated), ``"relu2"`` (ungated
    ReLU^2 MLP) or ``"attn"``."""

    cid: int
    kind: str
    T: int
    H: int
    r: int
    alpha: float
    dtype: str  # "f32" or "bf16"
    I: int = 0  # MLP intermediate size
    act: str = "swiglu"  # "swiglu" | "geglu_tanh"
    nf4: bool = False
    Nq: int = 0
    Nk: int = 0
    Nv: int = 0
    rms_inputs: bool = True  # X / dY rows RMS-normalised (RMSNorm-output stand-in)
    lora_dtype: str = ""  # "f32": adapters stay fp32 with bf16 inputs (fp32 LoRA-gradient mode)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return self.alpha / self.r

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    def flops(self) -> float:
        """Algorithmic flops of one forward+backward (no base-weight gradient)."""
        r = self.r
        if self.kind == "mlp":
            H, I = self.H, self.I
            return float(self.T) * (12 * H * I + 18 * r * (H + I))
        if self.kind == "relu2":  # up and down: 2 forward + 2 backward GEMMs, 2 adapters
            H, I = self.H, self.I
            return float(self.T) * (8 * H * I + 12 * r * (H + I))
        H = self.H
        tot = 0
        for n_out in (self.Nq, self.Nk, self.Nv):
            tot += 4 * H * n_out + 6 * r * (H + n_out)
        tot += 4 * self.Nq * H + 6 * r * (self.Nq + H)  # O: Nq -> H
        return float(self.T) * tot

    def with_(self, **kw) -> "WorkloadConfig":
        return replace(self, **kw)


CONFIGS = {
    1: WorkloadConfig(1, "mlp", T=128, H=256, I=704, r=8, alpha=16, dtype="f32",
                      act="swiglu", rms_inputs=False,
                      note="tiny SwiGLU LoRA-MLP, fp32 (batch 2 x seq 64)"),
    2: WorkloadConfig(2, "mlp", T=8192, H=4096, I=14336, r=16, alpha=32, dtype="bf16",
                      act="swiglu",
                      note="Llama-3-8B-shaped SwiGLU LoRA-MLP (4 x 2048 tokens)"),
    3: WorkloadConfig(3, "mlp", T=8192, H=3072, I=24576, r=16, alpha=16, dtype="bf16",
                      act="geglu_tanh", note="Gemma-style GeGLU-tanh LoRA-MLP"),
    4: WorkloadConfig(4, "mlp", T=8192, H=4096, I=14336, r=16, alpha=32, dtype="bf16",
                      act="swiglu", nf4=True,
                      note="QLoRA (NF4 base) SwiGLU LoRA-MLP, Llama-3-8B shape"),
    5: WorkloadConfig(5, "attn", T=8192, H=4096, r=16, alpha=32, dtype="bf16",
                      Nq=4096, Nk=1024, Nv=1024,
                      note="LoRA Q/K/V + O projections, Llama-3-8B attention shape"),
    6: WorkloadConfig(6, "relu2", T=8192, H=4096, I=21504, r=16, alpha=32, dtype="bf16",
                      note="Nemotron-H-8B-like ReLU^2 LoRA-MLP (4 x 2048 tokens)"),
}


def _normal(seed, name, shape, std):
    g = rng_for(seed, name)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _uniform(seed, name, shape, bound):
    g = rng_for(seed, name)
    return g.uniform(-bound, bound, size=shape).astype(np.float32)


def _rms_rows(x):
    ms = np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True)
    return (x / np.sqrt(ms + 1e-6)).astype(np.float32)


def _finish(x, cfg):
    return bf16_round(x) if cfg.dtype == "bf16" else np.ascontiguousarray(x, np.float32)


def make_proj(cfg: WorkloadConfig, prefix: str, n_in: int, n_out: int, seed=None):
    """Base weight and adapters of one projection: dict(W, A, B, s)."""
    seed = cfg.seed if seed is None else seed
    W = _normal(seed, prefix + ".W", (n_in, n_out), 1.0 / np.sqrt(n_in))
    A = _uniform(seed, prefix + ".A", (n_in, cfg.r), 1.0 / np.sqrt(n_in))
    B = _normal(seed, prefix + ".B", (cfg.r, n_out), 0.02)
    if cfg.lora_dtype == "f32":
        A, B = (np.ascontiguousarray(x, np.float32) for x in (A, B))
    else:
        A, B = _finish(A, cfg), _finish(B, cfg)
    return dict(W=_finish(W, cfg), A=A, B=B, s=float(cfg.scale))


def make_activation(cfg, name, T, n, seed=None, rms=None):
    seed = cfg.seed if seed is None else seed
    rms = cfg.rms_inputs if rms is None else rms
    x = _normal(seed, name, (T, n), 1.0)
    if rms and T > 0:
        x = _rms_rows(x)
    return _finish(x, cfg)


def make_mlp_inputs(cfg: WorkloadConfig, seed=None, T=None):
    """X, dY and the gate/up/down projections of one LoRA MLP block."""
    T = cfg.T if T is None else T
    out = dict(
        X=make_activation(cfg, "X", T, cfg.H, seed),
        dY=make_activation(cfg, "dY", T, cfg.H, seed),
        gate=make_proj(cfg, "gate", cfg.H, cfg.I, seed),
        up=make_proj(cfg, "up", cfg.H, cfg.I, seed),
        down=make_proj(cfg, "down", cfg.I, cfg.H, seed),
    )
    return out


def make_relu2_inputs(cfg: WorkloadConfig, seed=None, T=None):
    """X, dY and the up/down projections of one ungated ReLU^2 LoRA MLP."""
    T = cfg.T if T is None else T
    return dict(
        X=make_activation(cfg, "X", T, cfg.H, seed),
        dY=make_activation(cfg, "dY", T, cfg.H, seed),
        up=make_proj(cfg, "up", cfg.H, cfg.I, seed),
        down=make_proj(cfg, "down", cfg.I, cfg.H, seed),
    )


def make_inputs(cfg: WorkloadConfig, seed=None, T=None):
    """The inputs of any configuration, by its kind."""
    return {"mlp": make_mlp_inputs, "relu2": make_relu2_inputs, "attn": make_attn_inputs}[cfg.kind](cfg, seed, T)


def make_attn_inputs(cfg: WorkloadConfig, seed=None, T=None):
    """X (shared by Q/K/V), X_o (attention output), the four projections and
    the upstream gradients dQ, dK, dV, dO (plain N(0,1))."""
    T = cfg.T if T is None else T
    H = cfg.H
    out = dict(
        X=make_activation(cfg, "X", T, H, seed),
        Xo=make_activation(cfg, "Xo", T, cfg.Nq, seed),
        q=make_proj(cfg, "q", H, cfg.Nq, seed),
        k=make_proj(cfg, "k", H, cfg.Nk, seed),
        v=make_proj(cfg, "v", H, cfg.Nv, seed),
        o=make_proj(cfg, "o", cfg.Nq, H, seed),
        dQ=make_activation(cfg, "dQ", T, cfg.Nq, seed, rms=False),
        dK=make_activation(cfg, "dK", T, cfg.Nk, seed, rms=False),
        dV=make_activation(cfg, "dV", T, cfg.Nv, seed, rms=False),
        dO=make_activation(cfg, "dO", T, H, seed, rms=False),
    )
    return out
