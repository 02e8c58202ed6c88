"""Full-size parity on the GPU benchmark shapes.

The same calls bench.py times (lora_mlp_fwd/bwd, lora_qkv_fwd/bwd,
lora_o_fwd/bwd, lora_nf4_quantize) run at full size on seeded inputs, and
every output tensor is compared with the fp32 CPU oracle on the same inputs:
max|err|/max|ref| <= 2e-2 (bf16 with fp32 accumulation); NF4 codes, q8, s2
and mu bit-exact.  Each test takes tens of seconds, mostly the oracle.
"""
import time

import numpy as np
import pytest

from oracle import lora as OL
from oracle import nf4 as ON
from workload import CONFIGS, make_attn_inputs, make_mlp_inputs, make_relu2_inputs
from _util import TOL, assert_close, dev, host, proj_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def say(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.fixture(scope="module")
def lm():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_mlp_amd

    adapter_mlp_amd.load()
    return adapter_mlp_amd


def _mlp_full(lm, cid, lora_dtype=""):
    import torch

    cfg = CONFIGS[cid].with_(lora_dtype=lora_dtype)
    say(f"config {cid}: generating inputs ({cfg.note}{', fp32 adapters' if lora_dtype else ''})")
    inp = make_mlp_inputs(cfg)
    nf4 = {}
    if cfg.nf4:
        for k in ("gate", "up", "down"):
            say(f"config {cid}: NF4-quantizing {k} on the GPU and in the oracle")
            w = lm.nf4_quantize(dev(inp[k]["W"]))
            torch.cuda.synchronize()
            q = ON.quantize(inp[k]["W"])
            assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), f"{k}: codes differ"
            assert np.array_equal(w.q8.cpu().numpy(), q["q8"]), f"{k}: q8 differ"
            assert np.array_equal(w.s2.cpu().numpy().view(np.uint32), q["s2"].view(np.uint32)), f"{k}: s2 differ"
            assert w.mu.cpu().numpy().view(np.uint32)[0] == np.float32(q["mu"]).view(np.uint32), f"{k}: mu"
            nf4[k] = w
            inp[k] = dict(inp[k], W=ON.dequantize(q, "bf16"))
    say(f"config {cid}: GPU forward + backward")
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k], "bf16", nf4=nf4.get(k), adapters=lora_dtype or None) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, cfg.act)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, cfg.act)
    torch.cuda.synchronize()
    if lora_dtype:
        # the oracle multiplies with the adapters as the mode casts them; the
        # mode's gradients are fp32
        assert all(t.dtype == torch.float32 for t in grads.values())
        for k in ("gate", "up", "down"):
            inp[k] = OL.to_compute_adapters(inp[k])
    got = dict(Y=host(Y), e=host(saved["e"]), g=host(saved["g"]), U=host(saved["U"]), dX=host(dX),
               **{k: host(v) for k, v in grads.items()})
    del X, dY, Y, saved, dX, grads
    torch.cuda.empty_cache()
    say(f"config {cid}: oracle forward")
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], cfg.act)
    say(f"config {cid}: oracle backward")
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], cfg.act)
    tol = TOL["bf16"]
    assert_close("Y", got["Y"], Yr, tol)
    assert_close("e", got["e"], sr["e"], tol)
    assert_close("g", got["g"], sr["g"], tol)
    assert_close("U", got["U"], np.concatenate([sr["U_g"], sr["U_u"], sr["U_d"]], axis=1), tol)
    assert_close("dX", got["dX"], gr["dX"], tol)
    for k_dev, k_ref in (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
                         ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, got[k_dev], gr[k_ref], tol)


def test_config2_llama3_8b_mlp_swiglu(lm):
    _mlp_full(lm, 2)


def test_config2_fp32_lora_gradients(lm):
    _mlp_full(lm, 2, lora_dtype="f32")


def test_config3_gemma_geglu_tanh(lm):
    _mlp_full(lm, 3)


def test_config4_qlora_nf4_mlp(lm):
    _mlp_full(lm, 4)


def test_config5_qkv_o(lm):
    import torch

    cfg = CONFIGS[5]
    say("config 5: generating inputs")
    inp = make_attn_inputs(cfg)
    X = dev(inp["X"])
    q, k, v, o = (proj_dev(inp[n]) for n in ("q", "k", "v", "o"))
    say("config 5: GPU forward + backward")
    Q, K, V, U = lm.qkv_fwd(X, q, k, v)
    dX, grads = lm.qkv_bwd(dev(inp["dQ"]), dev(inp["dK"]), dev(inp["dV"]), X, U, q, k, v)
    Xo = dev(inp["Xo"])
    Yo, Uo = lm.o_fwd(Xo, o)
    dXo, dAo, dBo = lm.o_bwd(dev(inp["dO"]), Xo, Uo, o)
    torch.cuda.synchronize()
    say("config 5: oracle")
    (Qr, Kr, Vr), sr = OL.qkv_fwd(inp["X"], inp["q"], inp["k"], inp["v"])
    gr = OL.qkv_bwd(inp["dQ"], inp["dK"], inp["dV"], inp["X"], sr, inp["q"], inp["k"], inp["v"])
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    gor = OL.o_bwd(inp["dO"], inp["Xo"], so, inp["o"])
    tol = TOL["bf16"]
    for name, a, b in (("Q", Q, Qr), ("K", K, Kr), ("V", V, Vr), ("O", Yo, Yr)):
        assert_close(name, host(a), b, tol)
    assert_close("U", host(U), np.concatenate([sr["U_q"], sr["U_k"], sr["U_v"]], axis=1), tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for n in ("dA_q", "dB_q", "dA_k", "dB_k", "dA_v", "dB_v"):
        assert_close(n, host(grads[n]), gr[n], tol)
    assert_close("dX_o", host(dXo), gor["dX"], tol)
    assert_close("dA_o", host(dAo), gor["dA"], tol)
    assert_close("dB_o", host(dBo), gor["dB"], tol)


def test_config6_relu2_mlp(lm):
    import torch

    cfg = CONFIGS[6]
    say(f"config 6: generating inputs ({cfg.note})")
    inp = make_relu2_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    up, down = (proj_dev(inp[k]) for k in ("up", "down"))
    say("config 6: GPU forward + backward")
    Y, saved = lm.relu2_mlp_fwd(X, up, down)
    dX, grads = lm.relu2_mlp_bwd(dY, X, saved, up, down)
    torch.cuda.synchronize()
    got = dict(Y=host(Y), u=host(saved["u"]), U=host(saved["U"]), dX=host(dX),
               **{k: host(v) for k, v in grads.items()})
    del X, dY, Y, saved, dX, grads
    torch.cuda.empty_cache()
    say("config 6: oracle")
    Yr, sr = OL.relu2_mlp_fwd(inp["X"], inp["up"], inp["down"])
    gr = OL.relu2_mlp_bwd(inp["dY"], inp["X"], sr, inp["up"], inp["down"])
    tol = TOL["bf16"]
    assert_close("Y", got["Y"], Yr, tol)
    assert_close("u", got["u"], sr["u"], tol)
    assert_close("U", got["U"], np.concatenate([sr["U_u"], sr["U_d"]], axis=1), tol)
    assert_close("dX", got["dX"], gr["dX"], tol)
    for k_dev, k_ref in (("dA_up", "dA_u"), ("dB_up", "dB_u"), ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, got[k_dev], gr[k_ref], tol)
