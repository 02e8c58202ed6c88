"""Forward GEMMs over the K-contiguous weight copies: with Wt = W^T (the
[n_out, n_in] layout of PyTorch's nn.Linear) given, the forward GEMMs of
every entry point read Wt through the NT kernels (checked in the library's
launch trace), and all results match the oracle and the same calls with W
alone.  A GEMM whose projections do not all carry Wt reads W."""
import dataclasses

import numpy as np
import pytest

from oracle import lora as OL
from workload import WorkloadConfig, make_attn_inputs, make_mlp_inputs, make_relu2_inputs
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


def _with_wt(p):
    return dataclasses.replace(p, Wt=p.W.t().contiguous())


def _traced(lm, fn):
    import torch

    lm.trace_begin("gemm")
    out = fn()
    torch.cuda.synchronize()
    return out, lm.trace_end()


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
@pytest.mark.parametrize("which", ["all", "down", "gate"])
def test_mlp_forward_over_wt(lm, act, which):
    """I = 1088 leaves a 64-column gate/up tile at the edge.  "gate": only
    gate has Wt, so gate/up reads W and down reads W too."""
    cfg = WorkloadConfig(120, "mlp", T=700, H=512, I=1088, r=16, alpha=32, dtype="bf16", act=act)
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    names = ("gate", "up", "down")
    base = [proj_dev(inp[k]) for k in names]
    sel = {"all": names, "down": ("down",), "gate": ("gate",)}[which]
    g, u, d = (_with_wt(p) if n in sel else p for n, p in zip(names, base))
    Y0, _ = lm.mlp_fwd(X, *base, act)
    (Y, saved), fams = _traced(lm, lambda: lm.mlp_fwd(X, g, u, d, act))
    assert ("gemm_nt_act_fwd" in fams) == (which == "all"), fams
    assert ("gemm_nt_store" in fams) == (which in ("all", "down")), fams
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, act)
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], act)
    tol = TOL["bf16"]
    assert_close("Y", host(Y), Yr, tol)
    assert_close("e", host(saved["e"]), sr["e"], tol)
    assert_close("g", host(saved["g"]), sr["g"], tol)
    assert_close("U", host(saved["U"]), np.concatenate([sr["U_g"], sr["U_u"], sr["U_d"]], axis=1), tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in MLP_GRADS:
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)
    assert_close("Y (Wt) vs Y (W)", host(Y), host(Y0), tol)


def test_relu2_forward_over_wt(lm):
    cfg = WorkloadConfig(121, "relu2", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16")
    inp = make_relu2_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    up, down = (_with_wt(proj_dev(inp[k])) for k in ("up", "down"))
    (Y, saved), fams = _traced(lm, lambda: lm.relu2_mlp_fwd(X, up, down))
    assert "gemm_nt_relu2_fwd" in fams and "gemm_nt_store" in fams, fams
    dX, grads = lm.relu2_mlp_bwd(dY, X, saved, up, down)
    Yr, sr = OL.relu2_mlp_fwd(inp["X"], inp["up"], inp["down"])
    gr = OL.relu2_mlp_bwd(inp["dY"], inp["X"], sr, inp["up"], inp["down"])
    tol = TOL["bf16"]
    assert_close("Y", host(Y), Yr, tol)
    assert_close("u", host(saved["u"]), sr["u"], tol)
    assert_close("U", host(saved["U"]), np.concatenate([sr["U_u"], sr["U_d"]], axis=1), tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in (("dA_up", "dA_u"), ("dB_up", "dB_u"), ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)


@pytest.mark.parametrize("T", [1, 257])
def test_qkv_o_forward_over_wt(lm, T):
    cfg = WorkloadConfig(122, "attn", T=T, H=512, r=16, alpha=32, dtype="bf16", Nq=512, Nk=192, Nv=128)
    inp = make_attn_inputs(cfg)
    X, Xo = dev(inp["X"]), dev(inp["Xo"])
    q, k, v, o = (_with_wt(proj_dev(inp[n])) for n in ("q", "k", "v", "o"))
    (Q, K, V, U), fams = _traced(lm, lambda: lm.qkv_fwd(X, q, k, v))
    (Yo, Uo), fo = _traced(lm, lambda: lm.o_fwd(Xo, o))
    assert "gemm_nt_store" in fams and "gemm_nt_store" in fo and "gemm_nn_store" not in fams, (fams, fo)
    (Qr, Kr, Vr), sr = OL.qkv_fwd(inp["X"], inp["q"], inp["k"], inp["v"])
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    tol = TOL["bf16"]
    for name, a, b in (("Q", Q, Qr), ("K", K, Kr), ("V", V, Vr), ("O", Yo, Yr), ("U_o", Uo, so["U"])):
        assert_close(name, host(a), b, tol)
    assert_close("U", host(U), np.concatenate([sr["U_q"], sr["U_k"], sr["U_v"]], axis=1), tol)


def test_o_forward_over_wt_tail_split(lm):
    """The NT store GEMM with a forced split over 280 tiles (256 whole, 24 split)."""
    cfg = WorkloadConfig(123, "attn", T=2560, H=7168, r=16, alpha=32, dtype="bf16", Nq=512, Nk=128, Nv=128)
    inp = make_attn_inputs(cfg)
    Xo = dev(inp["Xo"])
    o = _with_wt(proj_dev(inp["o"]))
    (Yo, Uo), fams = _traced(lm, lambda: lm.o_fwd(Xo, o, plan=[(8, 2)]))
    assert "gemm_nt_store" in fams, fams
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    assert_close("O", host(Yo), Yr, TOL["bf16"])
    assert_close("U_o", host(Uo), so["U"], TOL["bf16"])


def test_mlp_forward_over_wt_fp32_adapters(lm):
    """The fp32 LoRA-gradient mode stages bf16 copies of the adapters; the
    staged projections keep Wt."""
    cfg = WorkloadConfig(124, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act="swiglu",
                         lora_dtype="f32")
    inp = make_mlp_inputs(cfg)
    X = dev(inp["X"])
    g, u, d = (_with_wt(proj_dev(inp[k], adapters="f32")) for k in ("gate", "up", "down"))
    (Y, saved), fams = _traced(lm, lambda: lm.mlp_fwd(X, g, u, d, "swiglu"))
    assert "gemm_nt_act_fwd" in fams, fams
    cast = {k: OL.to_compute_adapters(inp[k]) for k in ("gate", "up", "down")}
    Yr, sr = OL.mlp_fwd(inp["X"], cast["gate"], cast["up"], cast["down"], "swiglu")
    assert_close("Y", host(Y), Yr, TOL["bf16"])
    assert_close("e", host(saved["e"]), sr["e"], TOL["bf16"])


def test_o_forward_noalloc_over_wt(lm):
    """The no-allocation forward with Wt equals lora_o_fwd with Wt, on two calls
    in a row, the second smaller."""
    import torch

    for T in (700, 129):
        cfg = WorkloadConfig(125, "attn", T=T, H=512, r=16, alpha=32, dtype="bf16", Nq=512, Nk=128, Nv=128)
        inp = make_attn_inputs(cfg)
        Xo = dev(inp["Xo"])
        o = _with_wt(proj_dev(inp["o"]))
        Y1, U1 = lm.o_fwd(Xo, o)
        Y2 = torch.empty_like(Y1)
        U2 = torch.empty_like(U1)
        lm.o_fwd_noalloc(Xo, o, Y=Y2, U=U2)
        torch.cuda.synchronize()
        Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
        assert_close("O noalloc", host(Y2), Yr, TOL["bf16"])
        assert_close("U noalloc", host(U2), so["U"], TOL["bf16"])
        assert_close("O noalloc vs o_fwd", host(Y2), host(Y1), TOL["bf16"])
