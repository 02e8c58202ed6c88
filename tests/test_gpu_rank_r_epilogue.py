"""The rank-r products of the MLP backward formed in the dh GEMM's epilogue.

For bf16 calls with rank <= 16, the epilogue that writes dg and de (du for
the ungated ReLU^2 MLP) also forms P = dZ B^T and dB = s U^T dZ from the bf16
gradients, as per-tile partial sums; one reduce launch ("rowcol_reduce")
finishes them, and no separate pass reads the gradients again.  The launch
trace shows which path ran; every result is compared with the oracle."""
import numpy as np
import pytest

from oracle import lora as OL
from oracle import nf4 as ON
from workload import WorkloadConfig, make_mlp_inputs, make_relu2_inputs
from _util import TOL, assert_close, dev, host, proj_dev

pytestmark = pytest.mark.gpu

MLP_GRADS = (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
             ("dA_down", "dA_d"), ("dB_down", "dB_d"))
RELU2_GRADS = (("dA_up", "dA_u"), ("dB_up", "dB_u"), ("dA_down", "dA_d"), ("dB_down", "dB_d"))


@pytest.fixture(scope="module")
def lm():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_mlp_amd

    adapter_mlp_amd.load()
    return adapter_mlp_amd


def _traced(lm, fn):
    import torch

    lm.trace_begin("")
    out = fn()
    torch.cuda.synchronize()
    return out, lm.trace_end()


def _check_path(fams, fused):
    """One rank-r pass over dY; with the fused products, only their reduce for
    the gradients the dh epilogue writes, else a second pass over them."""
    if fused:
        assert fams.get("rowcol", (0,))[0] == 1 and fams.get("rowcol_reduce", (0,))[0] == 1, fams
    else:
        assert fams.get("rowcol", (0,))[0] >= 2 and "rowcol_reduce" not in fams, fams


def _mlp(lm, cfg, act, nf4=False, fused=True):
    import torch

    inp = make_mlp_inputs(cfg)
    nf = {}
    if nf4:
        for k in ("gate", "up", "down"):
            w = lm.nf4_quantize(dev(inp[k]["W"]))
            q = ON.quantize(inp[k]["W"])
            torch.cuda.synchronize()
            assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), f"{k}: NF4 codes differ"
            nf[k] = w
            inp[k] = dict(inp[k], W=ON.dequantize(q, "bf16"))
    ad = cfg.lora_dtype or None
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k], nf4=nf.get(k), adapters=ad) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, act)
    (dX, grads), fams = _traced(lm, lambda: lm.mlp_bwd(dY, X, saved, g, u, d, act))
    _check_path(fams, fused)
    if ad:
        assert all(t.dtype == torch.float32 for t in grads.values())
        inp = dict(inp, **{k: OL.to_compute_adapters(inp[k]) for k in ("gate", "up", "down")})
    _, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], act)
    tol = TOL["bf16"]
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in MLP_GRADS:
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_mlp_rank_r_in_dh_epilogue(lm, act):
    """I = 1088: the last dh tile has one wavefront column of four inside I;
    T = 700 ends in a partial m-tile."""
    cfg = WorkloadConfig(130, "mlp", T=700, H=512, I=1088, r=16, alpha=32, dtype="bf16", act=act)
    _mlp(lm, cfg, act)


def test_mlp_rank_r_in_dh_epilogue_rank8(lm):
    """A rank below 16 (bf16 ranks are multiples of 8): rows of B past the
    rank read zero, the U columns past it belong to the next adapter and only
    reach sums that are not read."""
    cfg = WorkloadConfig(131, "mlp", T=333, H=256, I=640, r=8, alpha=17, dtype="bf16", act="swiglu")
    _mlp(lm, cfg, "swiglu")


def test_mlp_rank_r_in_dh_epilogue_single_tile(lm):
    """T below one m-tile and I of one dh tile: a single partial slice each way."""
    cfg = WorkloadConfig(132, "mlp", T=37, H=128, I=256, r=16, alpha=32, dtype="bf16", act="geglu_tanh")
    _mlp(lm, cfg, "geglu_tanh")


def test_mlp_rank_r_in_dh_epilogue_fp32_adapters(lm):
    cfg = WorkloadConfig(133, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act="swiglu",
                         lora_dtype="f32")
    _mlp(lm, cfg, "swiglu")


def test_mlp_rank_r_in_dh_epilogue_nf4(lm):
    cfg = WorkloadConfig(134, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act="swiglu", nf4=True)
    _mlp(lm, cfg, "swiglu", nf4=True)


def test_mlp_rank_24_keeps_the_pass(lm):
    cfg = WorkloadConfig(135, "mlp", T=300, H=256, I=640, r=24, alpha=24, dtype="bf16", act="swiglu")
    _mlp(lm, cfg, "swiglu", fused=False)


def test_relu2_rank_r_in_dh_epilogue(lm):
    import torch

    cfg = WorkloadConfig(136, "relu2", T=700, H=512, I=1088, r=16, alpha=32, dtype="bf16")
    inp = make_relu2_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    up, down = (proj_dev(inp[k]) for k in ("up", "down"))
    Y, saved = lm.relu2_mlp_fwd(X, up, down)
    (dX, grads), fams = _traced(lm, lambda: lm.relu2_mlp_bwd(dY, X, saved, up, down))
    torch.cuda.synchronize()
    _check_path(fams, True)
    _, sr = OL.relu2_mlp_fwd(inp["X"], inp["up"], inp["down"])
    gr = OL.relu2_mlp_bwd(inp["dY"], inp["X"], sr, inp["up"], inp["down"])
    tol = TOL["bf16"]
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in RELU2_GRADS:
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)


def test_mlp_rank_r_in_dh_epilogue_deterministic(lm):
    """The partial slices are added in a fixed order: two calls agree bit for bit."""
    import torch

    cfg = WorkloadConfig(137, "mlp", T=700, H=512, I=1088, r=16, alpha=32, dtype="bf16", act="swiglu")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, "swiglu")
    outs = []
    for _ in range(2):
        dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, "swiglu")
        torch.cuda.synchronize()
        outs.append((dX.clone(), {k: v.clone() for k, v in grads.items()}))
    assert torch.equal(outs[0][0], outs[1][0])
    for k in outs[0][1]:
        assert torch.equal(outs[0][1][k], outs[1][1][k]), k
