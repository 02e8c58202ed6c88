"""GEMM launch plans on the GPU: every tile-group size and forced split-K
factors give the oracle's results, and the tuner ("loralei" README, section
"Use": time a few valid tile configurations per GPU and shape, keep the
fastest in a cache) tunes a shape outside the benchmark configurations,
writes its JSON cache, reloads it and runs with the tuned plans."""
import numpy as np
import pytest

from oracle import lora as OL
from workload import WorkloadConfig, make_attn_inputs, make_mlp_inputs
from _util import TOL, assert_close, dev, host, proj_dev

pytestmark = pytest.mark.gpu

MLP_GRADS = (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
             ("dA_down", "dA_d"), ("dB_down", "dB_d"))


@pytest.fixture(scope="module")
def lm():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_mlp_amd

    adapter_mlp_amd.load()
    return adapter_mlp_amd


def _mlp_with_plans(lm, cfg, fwd_plan, bwd_plan):
    import torch

    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, cfg.act, plan=fwd_plan)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, cfg.act, plan=bwd_plan)
    torch.cuda.synchronize()
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], cfg.act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], cfg.act)
    tol = TOL["bf16"]
    print(f"  plans fwd {fwd_plan} bwd {bwd_plan}", flush=True)
    assert_close("Y", host(Y), Yr, tol)
    assert_close("e", host(saved["e"]), sr["e"], tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in MLP_GRADS:
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)


@pytest.mark.parametrize("fwd_plan,bwd_plan", [
    ([(1, 0), (32, 4)], [(32, 0), (1, 3)]),
    ([(2, 1), (16, 2)], [(16, 1), (2, 4)]),
    ([(8, 0), (4, 0)], [(4, 0), (8, 2)]),
])
def test_forced_plans_mlp(lm, fwd_plan, bwd_plan):
    cfg = WorkloadConfig(110, "mlp", T=700, H=512, I=1088, r=16, alpha=32, dtype="bf16", act="swiglu")
    _mlp_with_plans(lm, cfg, fwd_plan, bwd_plan)


def test_forced_plans_qkv_o(lm):
    import torch

    cfg = WorkloadConfig(111, "attn", T=700, H=512, r=16, alpha=32, dtype="bf16", Nq=512, Nk=192, Nv=128)
    inp = make_attn_inputs(cfg)
    X = dev(inp["X"])
    q, k, v = (proj_dev(inp[n]) for n in ("q", "k", "v"))
    Q, K, V, U = lm.qkv_fwd(X, q, k, v, plan=[(16, 1)])
    dX, grads = lm.qkv_bwd(*(dev(inp[n]) for n in ("dQ", "dK", "dV")), X, U, q, k, v, plan=[(2, 3)])
    Xo = dev(inp["Xo"])
    o = proj_dev(inp["o"])
    Yo, Uo = lm.o_fwd(Xo, o, plan=[(32, 2)])
    dXo, dAo, dBo = lm.o_bwd(dev(inp["dO"]), Xo, Uo, o, plan=[(1, 4)])
    torch.cuda.synchronize()
    (Qr, Kr, Vr), sr = OL.qkv_fwd(inp["X"], inp["q"], inp["k"], inp["v"])
    gr = OL.qkv_bwd(inp["dQ"], inp["dK"], inp["dV"], inp["X"], sr, inp["q"], inp["k"], inp["v"])
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    go = OL.o_bwd(inp["dO"], inp["Xo"], so, inp["o"])
    tol = TOL["bf16"]
    for name, a, b in (("Q", Q, Qr), ("K", K, Kr), ("V", V, Vr), ("dX", dX, gr["dX"]), ("O", Yo, Yr),
                       ("dX_o", dXo, go["dX"]), ("dA_o", dAo, go["dA"]), ("dB_o", dBo, go["dB"])):
        assert_close(name, host(a), b, tol)
    for n in ("dA_q", "dB_q", "dA_k", "dB_k", "dA_v", "dB_v"):
        assert_close(n, host(grads[n]), gr[n], tol)


def test_tune_mlp_new_shape_and_cache(lm, tmp_path):
    """T = 3000, H = 2560, I = 9728 (none of the benchmark shapes): tune,
    write the cache, reload it in a fresh PlanCache, run with the tuned plans
    and compare with the oracle."""
    import torch

    from adapter_mlp_amd import tune

    cfg = WorkloadConfig(112, "mlp", T=3000, H=2560, I=9728, r=16, alpha=32, dtype="bf16", act="swiglu")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    path = str(tmp_path / "plans.json")
    cache = tune.PlanCache(path)
    assert tune.mlp_plans(cache, X, g, u, d, cfg.act) is None
    plans = tune.tune_mlp(cache, X, dY, g, u, d, cfg.act)
    entry = cache.get(tune.mlp_key(cfg.T, cfg.H, cfg.I, cfg.r, cfg.act, 1, False), X.device)
    print(f"  tuned {plans}; ms {entry['ms']}", flush=True)
    reloaded = tune.mlp_plans(tune.PlanCache(path), X, g, u, d, cfg.act)
    assert reloaded == plans
    Y, saved = lm.mlp_fwd(X, g, u, d, cfg.act, plan=reloaded["fwd"])
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, cfg.act, plan=reloaded["bwd"])
    torch.cuda.synchronize()
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], cfg.act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], cfg.act)
    tol = TOL["bf16"]
    assert_close("Y", host(Y), Yr, tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in MLP_GRADS:
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)
    assert entry["ms"]["fwd"]["tuned"] <= entry["ms"]["fwd"]["default"]
    assert entry["ms"]["bwd"]["tuned"] <= entry["ms"]["bwd"]["default"]


def test_tail_split_o_fwd_and_qkv_dx(lm):
    """Split-K of only the tiles past the grid's last full round: H = 7168
    gives the O forward and the Q/K/V input-gradient GEMM 10 x 28 = 280
    tiles, so a split of 2 runs 256 tiles whole and splits the other 24.
    Both results (and those of every GEMM of the calls) against the oracle,
    and against the same calls without a split."""
    import torch

    cfg = WorkloadConfig(113, "attn", T=2560, H=7168, r=16, alpha=32, dtype="bf16", Nq=512, Nk=128, Nv=128)
    inp = make_attn_inputs(cfg)
    X, Xo = dev(inp["X"]), dev(inp["Xo"])
    q, k, v, o = (proj_dev(inp[n]) for n in ("q", "k", "v", "o"))
    Yo, Uo = lm.o_fwd(Xo, o, plan=[(8, 2)])
    Yo1, _ = lm.o_fwd(Xo, o, plan=[(8, 1)])
    Q, K, V, U = lm.qkv_fwd(X, q, k, v)
    dQ, dK, dV = (dev(inp[n]) for n in ("dQ", "dK", "dV"))
    dX, grads = lm.qkv_bwd(dQ, dK, dV, X, U, q, k, v, plan=[(8, 2)])
    dX1, _ = lm.qkv_bwd(dQ, dK, dV, X, U, q, k, v, plan=[(8, 1)])
    torch.cuda.synchronize()
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    (Qr, Kr, Vr), sr = OL.qkv_fwd(inp["X"], inp["q"], inp["k"], inp["v"])
    gr = OL.qkv_bwd(inp["dQ"], inp["dK"], inp["dV"], inp["X"], sr, inp["q"], inp["k"], inp["v"])
    tol = TOL["bf16"]
    assert_close("O", host(Yo), Yr, tol)
    assert_close("U_o", host(Uo), so["U"], tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for n in ("dA_q", "dB_q", "dA_k", "dB_k", "dA_v", "dB_v"):
        assert_close(n, host(grads[n]), gr[n], tol)
    # the split changes only the fp32 summation order of the split tiles' K parts
    assert_close("O split vs whole", host(Yo), host(Yo1), tol)
    assert_close("dX split vs whole", host(dX), host(dX1), tol)


@pytest.mark.parametrize("ksplit", [3, 4])
def test_tail_split_ragged(lm, ksplit):
    """A tail split over ragged edge tiles: T = 2660 and N = 7104 give
    11 x 28 = 308 tiles (the last m-tile 100 rows, the last n-tile 192
    columns), 256 computed whole and 52 split into 3 or 4 K parts."""
    import torch

    cfg = WorkloadConfig(114, "attn", T=2660, H=7104, r=16, alpha=32, dtype="bf16", Nq=512, Nk=128, Nv=128)
    inp = make_attn_inputs(cfg)
    Xo = dev(inp["Xo"])
    o = proj_dev(inp["o"])
    Yo, Uo = lm.o_fwd(Xo, o, plan=[(8, ksplit)])
    torch.cuda.synchronize()
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    tol = TOL["bf16"]
    assert_close("O", host(Yo), Yr, tol)
    assert_close("U_o", host(Uo), so["U"], tol)
