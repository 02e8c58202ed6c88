"""The Python binding checks every tensor against the call's shapes before it
hands pointers to the C ABI: shape, dtype, contiguity and device, including
the outputs, saved tensors and gradients a caller supplies.  Each mismatch
raises ValueError before the library is called; these tests run on CPU
tensors (a correct set of CPU tensors is refused last, because the library
runs on the GPU only)."""
import pytest
import torch

import adapter_mlp_amd as lm

T, H, I, r = 8, 64, 128, 8


def _proj(n_in, n_out, dtype=torch.bfloat16, ad=None):
    ad = ad or dtype
    return lm.Proj(A=torch.zeros(n_in, r, dtype=ad), B=torch.zeros(r, n_out, dtype=ad), scale=1.0,
                   W=torch.zeros(n_in, n_out, dtype=dtype))


def _mlp(dtype=torch.bfloat16, ad=None):
    return _proj(H, I, dtype, ad), _proj(H, I, dtype, ad), _proj(I, H, dtype, ad)


def _saved(dtype=torch.bfloat16):
    return dict(e=torch.zeros(T, I, dtype=dtype), g=torch.zeros(T, I, dtype=dtype), U=torch.zeros(T, 3 * r, dtype=dtype))


def test_correct_cpu_tensors_are_refused_as_not_on_gpu():
    X = torch.zeros(T, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU only"):
        lm.mlp_fwd(X, *_mlp())
    with pytest.raises(ValueError, match="GPU only"):
        lm.mlp_bwd(torch.zeros(T, H, dtype=torch.bfloat16), X, _saved(), *_mlp())


@pytest.mark.parametrize("case", ["noncontig_X", "short_dY", "bad_saved_U", "bf16_grad_in_f32lora",
                                  "wrong_W_shape", "transposed_W_view", "bad_A_rank", "mixed_adapter_dtypes",
                                  "W_dtype", "dX_shape", "Y_dtype"])
def test_mlp_mismatches_raise(case):
    X = torch.zeros(T, H, dtype=torch.bfloat16)
    dY = torch.zeros(T, H, dtype=torch.bfloat16)
    g, u, d = _mlp()
    saved = _saved()
    kw = {}
    fwd = False
    if case == "noncontig_X":
        X = torch.zeros(H, T, dtype=torch.bfloat16).t()
        fwd = True
    elif case == "short_dY":
        dY = torch.zeros(T - 1, H, dtype=torch.bfloat16)
    elif case == "bad_saved_U":
        saved["U"] = torch.zeros(T, 2 * r, dtype=torch.bfloat16)
    elif case == "bf16_grad_in_f32lora":
        g, u, d = _mlp(ad=torch.float32)
        kw["grads"] = {k: torch.zeros_like(getattr(p, ab), dtype=torch.bfloat16)
                       for k, p, ab in zip(("dA_gate", "dB_gate", "dA_up", "dB_up", "dA_down", "dB_down"),
                                           (g, g, u, u, d, d), "ABABAB")}
    elif case == "wrong_W_shape":
        u.W = torch.zeros(H, I + 64, dtype=torch.bfloat16)
    elif case == "transposed_W_view":
        # an nn.Linear weight [out, in] seen as [in, out]: right shape, not dense
        g.W = torch.zeros(I, H, dtype=torch.bfloat16).t()
    elif case == "bad_A_rank":
        d.A = torch.zeros(I, r + 8, dtype=torch.bfloat16)
    elif case == "mixed_adapter_dtypes":
        d.B = d.B.float()
    elif case == "W_dtype":
        d.W = d.W.float()
    elif case == "dX_shape":
        kw["dX"] = torch.zeros(T, H + 64, dtype=torch.bfloat16)
    elif case == "Y_dtype":
        kw["Y"] = torch.zeros(T, H, dtype=torch.float32)
        fwd = True
    with pytest.raises(ValueError):
        if fwd:
            lm.mlp_fwd(X, g, u, d, **kw)
        else:
            lm.mlp_bwd(dY, X, saved, g, u, d, **kw)


def test_relu2_qkv_o_mismatches_raise():
    X = torch.zeros(T, H, dtype=torch.bfloat16)
    up, down = _proj(H, I), _proj(I, H)
    saved = dict(u=torch.zeros(T, I, dtype=torch.bfloat16), U=torch.zeros(T, r, dtype=torch.bfloat16))  # U too narrow
    with pytest.raises(ValueError, match="U"):
        lm.relu2_mlp_bwd(X.clone(), X, saved, up, down)
    q, k, v = _proj(H, 128), _proj(H, 64), _proj(H, 64)
    with pytest.raises(ValueError, match="dK"):
        lm.qkv_bwd(torch.zeros(T, 128, dtype=torch.bfloat16), torch.zeros(T, 128, dtype=torch.bfloat16),
                   torch.zeros(T, 64, dtype=torch.bfloat16), X, torch.zeros(T, 3 * r, dtype=torch.bfloat16), q, k, v)
    with pytest.raises(ValueError, match="Q"):
        lm.qkv_fwd(X, q, k, v, out=[torch.zeros(T, 64, dtype=torch.bfloat16), torch.zeros(T, 64, dtype=torch.bfloat16),
                                    torch.zeros(T, 64, dtype=torch.bfloat16)])
    o = _proj(H, 128)
    with pytest.raises(ValueError, match="dA"):
        lm.o_bwd(torch.zeros(T, 128, dtype=torch.bfloat16), X, torch.zeros(T, r, dtype=torch.bfloat16), o,
                 dA=torch.zeros(H, r, dtype=torch.float32))
    with pytest.raises(ValueError, match="ws"):
        lm.o_fwd(X, o, ws=torch.zeros(1024, dtype=torch.uint8)[::2])


def test_nf4_weight_arrays_checked():
    n_in, n_out = 128, 128
    w = lm.NF4Weight(codes=torch.zeros(n_in * n_out // 2, dtype=torch.uint8),
                     q8=torch.zeros(n_in * n_out // 64, dtype=torch.int8),
                     s2=torch.zeros(n_in * n_out // 16384, dtype=torch.float32),
                     mu=torch.zeros(1, dtype=torch.float32), rows=n_in, cols=n_out)
    X = torch.zeros(T, n_in, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU only"):
        lm.nf4_gemm(X, w)
    bad = lm.NF4Weight(codes=w.codes[:-16], q8=w.q8, s2=w.s2, mu=w.mu, rows=n_in, cols=n_out)
    with pytest.raises(ValueError, match="codes"):
        lm.nf4_gemm(X, bad)
    with pytest.raises(ValueError, match="X"):
        lm.nf4_gemm(torch.zeros(T, n_in + 64, dtype=torch.bfloat16), w)
    p = lm.Proj(A=torch.zeros(n_in, r, dtype=torch.bfloat16), B=torch.zeros(r, n_out, dtype=torch.bfloat16),
                scale=1.0, nf4=lm.NF4Weight(codes=w.codes, q8=w.q8.to(torch.uint8), s2=w.s2, mu=w.mu, rows=n_in,
                                            cols=n_out))
    with pytest.raises(ValueError, match="q8"):
        lm.o_fwd(X, p)


def test_wt_checked():
    """Wt is the dense weight stored [n_out, n_in]: the wrong shape, a
    non-contiguous view, or Wt beside an NF4 weight raise before any call."""
    X = torch.zeros(T, H, dtype=torch.bfloat16)
    o = _proj(H, 128)
    o.Wt = torch.zeros(H, 128, dtype=torch.bfloat16)  # [n_in, n_out]: transposed shape
    with pytest.raises(ValueError, match="Wt"):
        lm.o_fwd(X, o)
    o.Wt = torch.zeros(H, 128, dtype=torch.bfloat16).t()  # right shape, not contiguous
    with pytest.raises(ValueError, match="Wt"):
        lm.o_fwd(X, o)
    o2 = lm.Proj(A=o.A, B=o.B, scale=1.0, nf4=object(), Wt=torch.zeros(128, H, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="Wt"):
        lm.o_fwd(X, o2)
