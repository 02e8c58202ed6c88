"""Measured per-shape GEMM launch plans with an on-disk cache.

The QLoRA path of the "loralei" README (section "Use") warms each distinct
shape, times a small set of valid tile configurations and keeps the fastest
per GPU and shape in a JSON cache, falling back to a conservative default on
a miss.  The C library keeps no state, so the cache lives here, with the
caller: a plan (``lora_plan`` in the C header) is passed with each call, and
``None`` keeps the library's defaults (its analytic split-K model and tile
groups of 4 or 8).

What is tuned, per GEMM of a call:
  * ``group``  -- m-tiles per group of the XCD-aware tile order, which sets
    how many activation and weight panels the tiles resident on one XCD
    share in its L2;
  * ``ksplit`` -- the split-K factor of a plain-store GEMM (fp32 partials
    added in a fixed order), which fills a poorly filled last wave of tiles.
Plans never change what is computed, only the order of the work; a split-K
plan changes the fp32 summation order of the split GEMM.

Typical use::

    from adapter_mlp_amd import tune
    cache = tune.PlanCache()                       # JSON file, see PlanCache
    plans = tune.mlp_plans(cache, X, gate, up, down, act)   # cached or None
    if plans is None:
        plans = tune.tune_mlp(cache, X, dY, gate, up, down, act)
    Y, saved = mlp_fwd(X, gate, up, down, act, plan=plans["fwd"])
    dX, grads = mlp_bwd(dY, X, saved, gate, up, down, act, plan=plans["bwd"])
"""
from __future__ import annotations

import json
import os
import statistics
import tempfile


GROUPS = (2, 4, 8, 16)
KSPLITS = (1, 2, 3, 4)
DEFAULT_CACHE = os.path.join(os.path.expanduser("~"), ".cache", "adapter_mlp_amd", "plans.json")


def device_key(device=None) -> str:
    """Identifies the GPU a plan was measured on: architecture, compute-unit
    count and product name."""
    import torch

    p = torch.cuda.get_device_properties(device if device is not None else torch.cuda.current_device())
    arch = getattr(p, "gcnArchName", "unknown")
    return f"{arch}:{p.multi_processor_count}cu:{p.name}"


class PlanCache:
    """JSON cache of measured plans, keyed by device and shape.  The file is
    ``path``, else $LORA_MI355X_PLAN_CACHE, else ~/.cache/adapter_mlp_amd/plans.json;
    it is read once and rewritten atomically by put()."""

    VERSION = 1

    def __init__(self, path: str | None = None):
        self.path = path or os.environ.get("LORA_MI355X_PLAN_CACHE") or DEFAULT_CACHE
        self.data = {"version": self.VERSION, "devices": {}}
        if os.path.exists(self.path):
            with open(self.path) as f:
                d = json.load(f)
            if d.get("version") == self.VERSION:
                self.data = d

    def get(self, shape_key: str, device=None):
        return self.data["devices"].get(device_key(device), {}).get(shape_key)

    def put(self, shape_key: str, entry: dict, device=None) -> None:
        self.data["devices"].setdefault(device_key(device), {})[shape_key] = entry
        d = os.path.dirname(os.path.abspath(self.path))
        os.makedirs(d, exist_ok=True)
        fd, tmp = tempfile.mkstemp(dir=d, prefix=".plans.", suffix=".json")
        with os.fdopen(fd, "w") as f:
            json.dump(self.data, f, indent=1, sort_keys=True)
        os.replace(tmp, self.path)


def _as_plan(entry):
    return [tuple(e) for e in entry] if entry is not None else None


def _time_ms(run, plan, reps: int, rounds: int = 3) -> float:
    """Median over `rounds` of the mean time of `reps` calls (HIP events on
    the current stream, after one untimed call)."""
    import torch

    run(plan)
    times = []
    for _ in range(rounds):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run(plan)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    return statistics.median(times)


def _default_of(i, gemms):
    """The candidate equal to the library's default for GEMM i: tile groups
    of 4 for the first GEMM of a two-GEMM call (an activation epilogue), 8
    otherwise, with the split-K model."""
    return (4, 0) if (len(gemms) == 2 and i == 0) else (8, 0)


def tune_call(run, gemms, reps: int = 3):
    """Tunes the GEMMs of one call.  run(plan) runs the call with a plan;
    gemms lists, per GEMM in launch order, (splittable, k_steps).  Each GEMM
    is tuned with the others at their defaults: first the tile group (split
    K as the library's model decides), then, for a splittable GEMM, the
    split factor under the best group.  Returns (plan, timings) with the
    default plan's time under the key "default"."""
    import time

    import torch

    n = len(gemms)
    base = [(0, 0)] * n
    # warm the clocks for at least 0.1 s before the first measurement
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            run(base)
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > 0.1:
            break
    timings = {"default": _time_ms(run, base, reps)}
    best = list(base)
    for i, (splittable, ksteps) in enumerate(gemms):
        cands = [(g, 0) for g in GROUPS]
        scores = {}
        for c in cands:
            plan = list(base)
            plan[i] = c
            scores[c] = _time_ms(run, plan, reps)
        g_best = min(scores, key=scores.get)
        if splittable:
            for k in KSPLITS:
                if k > ksteps:
                    break
                c = (g_best[0], k)
                plan = list(base)
                plan[i] = c
                scores[c] = _time_ms(run, plan, reps)
        pick = min(scores, key=scores.get)
        # keep the default unless a candidate is measurably faster (1%) than
        # the same GEMM at its default
        ref = scores.get(_default_of(i, gemms), timings["default"])
        best[i] = pick if scores[pick] < 0.99 * min(ref, timings["default"]) else (0, 0)
        timings.update({f"gemm{i}:{c[0]}/{c[1]}": t for c, t in scores.items()})
    # the baseline is the faster of two measurements, before and after the candidates
    timings["default"] = min(timings["default"], _time_ms(run, base, reps))
    if best == base:
        timings["tuned"] = timings["default"]
        return best, timings
    timings["tuned"] = _time_ms(run, best, reps)
    if timings["tuned"] > timings["default"]:
        best = list(base)
        timings["tuned"] = timings["default"]
    return best, timings


# ---------------------------------------------------------------------------
# Gated MLP
# ---------------------------------------------------------------------------

def _base(nf4, wt) -> str:
    """Base weights of a key: NF4, dense, or dense with the nn.Linear-layout
    copies (Wt), whose forward GEMMs run other kernels."""
    return "nf4" if nf4 else ("dense_wt" if wt else "dense")


def _has_wt(projs) -> bool:
    return all(getattr(p, "Wt", None) is not None for p in projs)


def mlp_key(T, H, I, r, act, dtype_code, nf4, wt=False) -> str:
    return f"mlp:T={T}:H={H}:I={I}:r={r}:act={act}:dtype={dtype_code}:base={_base(nf4, wt)}"


def _mlp_shape(X, gate, up, down, act):
    from . import _call_dtype

    T, H = X.shape
    I, r = gate.B.shape[1], gate.A.shape[1]
    wt = _has_wt((gate, up, down))
    return T, H, I, r, mlp_key(T, H, I, r, act, _call_dtype(X, (gate,)), gate.nf4 is not None, wt)


def mlp_plans(cache: PlanCache, X, gate, up, down, act="swiglu"):
    """The cached plans {"fwd": plan, "bwd": plan} of this shape on this GPU,
    or None (a miss: call with plan=None for the library's defaults)."""
    *_, key = _mlp_shape(X, gate, up, down, act)
    e = cache.get(key, X.device)
    return None if e is None else {"fwd": _as_plan(e["fwd"]), "bwd": _as_plan(e["bwd"])}


def tune_mlp(cache: PlanCache, X, dY, gate, up, down, act="swiglu", reps: int = 3):
    """Times plan candidates of lora_mlp_fwd (gate/up, down) and lora_mlp_bwd
    (dh, dX) on these tensors, stores the winners in the cache and returns
    {"fwd": plan, "bwd": plan}."""
    from . import mlp_bwd, mlp_fwd

    T, H, I, r, key = _mlp_shape(X, gate, up, down, act)
    dense_down, dense_gu = down.nf4 is None, gate.nf4 is None
    Y, saved = mlp_fwd(X, gate, up, down, act)
    fwd, tf = tune_call(lambda p: mlp_fwd(X, gate, up, down, act, Y=Y, saved=saved, plan=p),
                        [(False, H // 64 + 1), (dense_down, I // 64 + 1)], reps)
    dX, grads = mlp_bwd(dY, X, saved, gate, up, down, act)
    bwd, tb = tune_call(lambda p: mlp_bwd(dY, X, saved, gate, up, down, act, dX=dX, grads=grads, plan=p),
                        [(False, H // 64 + 1), (dense_gu, 2 * I // 64 + 1)], reps)
    entry = {"fwd": fwd, "bwd": bwd, "ms": {"fwd": tf, "bwd": tb}}
    cache.put(key, entry, X.device)
    return {"fwd": _as_plan(fwd), "bwd": _as_plan(bwd)}


# ---------------------------------------------------------------------------
# Q/K/V and single projections
# ---------------------------------------------------------------------------

def qkv_key(T, H, Ns, r, dtype_code, nf4, wt=False) -> str:
    return f"qkv:T={T}:H={H}:N={Ns[0]},{Ns[1]},{Ns[2]}:r={r}:dtype={dtype_code}:base={_base(nf4, wt)}"


def tune_qkv(cache: PlanCache, X, dQ, dK, dV, q, k, v, reps: int = 3):
    """Tunes lora_qkv_fwd (one three-region GEMM, tile group only) and
    lora_qkv_bwd (the dX GEMM); stores and returns {"fwd": plan, "bwd": plan}."""
    from . import _call_dtype, qkv_bwd, qkv_fwd

    T, H = X.shape
    Ns = [p.B.shape[1] for p in (q, k, v)]
    r = q.A.shape[1]
    key = qkv_key(T, H, Ns, r, _call_dtype(X, (q,)), q.nf4 is not None, _has_wt((q, k, v)))
    Q, K, V, U = qkv_fwd(X, q, k, v)
    fwd, tf = tune_call(lambda p: qkv_fwd(X, q, k, v, out=[Q, K, V], U=U, plan=p), [(False, H // 64 + 1)], reps)
    dX, grads = qkv_bwd(dQ, dK, dV, X, U, q, k, v)
    bwd, tb = tune_call(lambda p: qkv_bwd(dQ, dK, dV, X, U, q, k, v, dX=dX, grads=grads, plan=p),
                        [(q.nf4 is None, sum(Ns) // 64 + 1)], reps)
    cache.put(key, {"fwd": fwd, "bwd": bwd, "ms": {"fwd": tf, "bwd": tb}}, X.device)
    return {"fwd": _as_plan(fwd), "bwd": _as_plan(bwd)}


def o_key(T, K, N, r, dtype_code, nf4, wt=False) -> str:
    return f"o:T={T}:K={K}:N={N}:r={r}:dtype={dtype_code}:base={_base(nf4, wt)}"


def tune_o(cache: PlanCache, X, dY, o, reps: int = 3):
    """Tunes lora_o_fwd and lora_o_bwd (one GEMM each); stores and returns
    {"fwd": plan, "bwd": plan}."""
    from . import _call_dtype, o_bwd, o_fwd

    T, K = X.shape
    N, r = o.B.shape[1], o.A.shape[1]
    key = o_key(T, K, N, r, _call_dtype(X, (o,)), o.nf4 is not None, _has_wt((o,)))
    Y, U = o_fwd(X, o)
    fwd, tf = tune_call(lambda p: o_fwd(X, o, Y=Y, U=U, plan=p), [(o.nf4 is None, K // 64 + 1)], reps)
    dX, dA, dB = o_bwd(dY, X, U, o)
    bwd, tb = tune_call(lambda p: o_bwd(dY, X, U, o, dX=dX, dA=dA, dB=dB, plan=p), [(o.nf4 is None, N // 64 + 1)],
                        reps)
    cache.put(key, {"fwd": fwd, "bwd": bwd, "ms": {"fwd": tf, "bwd": tb}}, X.device)
    return {"fwd": _as_plan(fwd), "bwd": _as_plan(bwd)}


def cached(cache: PlanCache, key: str, device=None):
    """{"fwd": plan, "bwd": plan} stored under `key` for this GPU, or None."""
    e = cache.get(key, device)
    return None if e is None else {"fwd": _as_plan(e["fwd"]), "bwd": _as_plan(e["bwd"])}


__all__ = ["PlanCache", "device_key", "tune_call", "mlp_key", "mlp_plans", "tune_mlp", "qkv_key", "tune_qkv",
           "o_key", "tune_o", "cached"]
