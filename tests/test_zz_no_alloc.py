"""lora_o_fwd_noalloc, the O forward that allocates nothing (its scratch is a
static per-GPU array), against lora_o_fwd and the oracle on the same seeded
inputs: two calls in a row, the second with fewer tokens, in bf16, fp32 and
the fp32 LoRA-gradient mode; a call whose scratch need exceeds the static
array is refused with LORA_EWORKSPACE and writes nothing."""
import numpy as np
import pytest

from oracle import lora as OL
from workload import WorkloadConfig, make_attn_inputs
from _util import TOL, assert_close, dev, host, proj_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lm():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_mlp_amd

    adapter_mlp_amd.load()
    return adapter_mlp_amd


def _run(lm, cfg, T):
    import torch

    inp = make_attn_inputs(cfg, T=T)
    dt = cfg.dtype
    ad = cfg.lora_dtype or None
    Xo = dev(inp["Xo"], dt)
    o = proj_dev(inp["o"], dt, adapters=ad)
    Y = torch.full((T, cfg.H), 7.0, dtype=Xo.dtype, device="cuda:0")
    U = torch.full((T, cfg.r), 7.0, dtype=Xo.dtype, device="cuda:0")
    lm.o_fwd_noalloc(Xo, o, Y=Y, U=U)
    Y2, U2 = lm.o_fwd(Xo, o)
    torch.cuda.synchronize()
    p = OL.to_compute_adapters(inp["o"]) if ad else inp["o"]
    Yr, so = OL.o_fwd(inp["Xo"], p)
    tol = TOL[dt]
    print(f"  T = {T}, {dt}{', fp32 adapters' if ad else ''}", flush=True)
    assert_close("Y vs o_fwd", host(Y), host(Y2), tol)
    assert_close("U vs o_fwd", host(U), host(U2), tol)
    assert_close("Y vs oracle", host(Y), Yr, tol)
    assert_close("U vs oracle", host(U), so["U"], tol)
    return Y, Y2


@pytest.mark.parametrize("dt,lora_dtype", [("bf16", ""), ("f32", ""), ("bf16", "f32")])
def test_noalloc_o_fwd_two_calls(lm, dt, lora_dtype):
    import torch

    cfg = WorkloadConfig(108, "attn", T=3000, H=768, r=16, alpha=32, dtype=dt, Nq=512, Nk=64, Nv=64,
                         lora_dtype=lora_dtype)
    Y, Y2 = _run(lm, cfg, 3000)
    if dt == "bf16":
        # K = 512 leaves no room for a split-K in lora_o_fwd: same kernels, same order
        assert torch.equal(Y, Y2)
    _run(lm, cfg, 257)


def test_noalloc_o_fwd_refuses_beyond_its_scratch(lm):
    import torch

    T, K, N, r = 300_000, 64, 64, 8  # 128 bytes per token alone exceed 32 MiB
    X = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda:0")
    o = lm.Proj(A=torch.zeros((K, r), dtype=torch.bfloat16, device="cuda:0"),
                B=torch.zeros((r, N), dtype=torch.bfloat16, device="cuda:0"), scale=1.0,
                W=torch.zeros((K, N), dtype=torch.bfloat16, device="cuda:0"))
    Y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device="cuda:0")
    U = torch.full((T, r), 7.0, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(lm.LoraError) as ei:
        lm.o_fwd_noalloc(X, o, Y=Y, U=U)
    assert ei.value.status == 5  # LORA_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.all(Y == 7.0) and torch.all(U == 7.0)
