"""Pins of the LoRA oracle against what the pages and the mathematics fix.

Each check is independent of the oracle's own formulas: finite differences of
the forward (for every analytic gradient), the merged-weight closed form (a
different association of the adapter term), exact zeros from the special
cases B = 0 / A = 0 / s = 0, bitwise identity of the hoisted product (the
unsloth commit message states the hoist changes no bit), row independence
under a token permutation, and textbook values of the activations.
"""
import numpy as np
import pytest
from scipy import special

from oracle import lora as L

F64 = np.float64


def _proj(rng, n_in, n_out, r, s, dtype=F64, zero_B=False, zero_A=False):
    W = rng.standard_normal((n_in, n_out)) / np.sqrt(n_in)
    A = rng.uniform(-1, 1, (n_in, r)) / np.sqrt(n_in)
    B = rng.standard_normal((r, n_out)) * 0.5
    if zero_B:
        B = np.zeros_like(B)
    if zero_A:
        A = np.zeros_like(A)
    return dict(W=W.astype(dtype), A=A.astype(dtype), B=B.astype(dtype), s=s)


def _mlp_problem(seed=0, T=3, H=8, I=12, r=2, s=1.5, **kw):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, H))
    dY = rng.standard_normal((T, H))
    gate = _proj(rng, H, I, r, s, **kw)
    up = _proj(rng, H, I, r, s * 0.5, **kw)
    down = _proj(rng, I, H, r, s * 2.0, **kw)
    return X, dY, gate, up, down


def _central_fd(f, x, eps=1e-6):
    """d f / d x for a scalar function f of array x (modified in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def _assert_grad(analytic, numeric, what):
    scale = max(np.abs(numeric).max(), 1e-12)
    err = np.abs(analytic - numeric).max() / scale
    assert err <= 1e-6, f"{what}: rel err {err:.3e}"


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_mlp_gradients_match_finite_differences(act):
    X, dY, gate, up, down = _mlp_problem()

    def loss():
        Y, _ = L.mlp_fwd(X, gate, up, down, act)
        return float(np.sum(Y * dY))

    Y, saved = L.mlp_fwd(X, gate, up, down, act)
    g = L.mlp_bwd(dY, X, saved, gate, up, down, act)
    _assert_grad(g["dX"], _central_fd(loss, X), "dX")
    for name, p in (("g", gate), ("u", up), ("d", down)):
        _assert_grad(g["dA_" + name], _central_fd(loss, p["A"]), "dA_" + name)
        _assert_grad(g["dB_" + name], _central_fd(loss, p["B"]), "dB_" + name)


def test_qkv_and_o_gradients_match_finite_differences():
    rng = np.random.default_rng(1)
    T, H, r = 4, 8, 3
    X = rng.standard_normal((T, H))
    q, k, v = _proj(rng, H, 8, r, 2.0), _proj(rng, H, 4, r, 0.5), _proj(rng, H, 4, r, 1.0)
    dQ, dK, dV = (rng.standard_normal((T, n)) for n in (8, 4, 4))

    def loss():
        (Q, K, V), _ = L.qkv_fwd(X, q, k, v)
        return float(np.sum(Q * dQ) + np.sum(K * dK) + np.sum(V * dV))

    _, saved = L.qkv_fwd(X, q, k, v)
    g = L.qkv_bwd(dQ, dK, dV, X, saved, q, k, v)
    _assert_grad(g["dX"], _central_fd(loss, X), "dX")
    for name, p in (("q", q), ("k", k), ("v", v)):
        _assert_grad(g["dA_" + name], _central_fd(loss, p["A"]), "dA_" + name)
        _assert_grad(g["dB_" + name], _central_fd(loss, p["B"]), "dB_" + name)

    o = _proj(rng, 8, H, r, 2.0)
    Xo = rng.standard_normal((T, 8))
    dO = rng.standard_normal((T, H))

    def loss_o():
        Y, _ = L.o_fwd(Xo, o)
        return float(np.sum(Y * dO))

    _, so = L.o_fwd(Xo, o)
    go = L.o_bwd(dO, Xo, so, o)
    _assert_grad(go["dX"], _central_fd(loss_o, Xo), "dX_o")
    _assert_grad(go["dA"], _central_fd(loss_o, o["A"]), "dA_o")
    _assert_grad(go["dB"], _central_fd(loss_o, o["B"]), "dB_o")


def test_merged_weight_closed_form_single_projection():
    """Forward: X@W + s*(X@A)@B == X@(W + s*A@B) (the merge that the loralei
    README offers as merge_lora).  Backward: with G = X.T @ dZ the gradient of
    a full weight, dA = s*G@B.T and dB = s*A.T@G."""
    rng = np.random.default_rng(2)
    T, n_in, n_out, r, s = 7, 10, 6, 3, 1.75
    X = rng.standard_normal((T, n_in))
    dZ = rng.standard_normal((T, n_out))
    p = _proj(rng, n_in, n_out, r, s)
    Z, U = L.proj_fwd(X, p["W"], p["A"], p["B"], s)
    merged = p["W"] + s * (p["A"] @ p["B"])
    np.testing.assert_allclose(Z, X @ merged, rtol=0, atol=1e-12 * np.abs(Z).max())
    dX, dA, dB = L.proj_bwd(dZ, X, p["W"], p["A"], p["B"], s, U)
    G = X.T @ dZ
    np.testing.assert_allclose(dA, s * G @ p["B"].T, rtol=0, atol=1e-12 * np.abs(dA).max())
    np.testing.assert_allclose(dB, s * p["A"].T @ G, rtol=0, atol=1e-12 * np.abs(dB).max())
    np.testing.assert_allclose(dX, dZ @ merged.T, rtol=0, atol=1e-12 * np.abs(dX).max())


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_mlp_equals_base_mlp_on_merged_weights(act):
    X, dY, gate, up, down = _mlp_problem(seed=3, T=5, H=8, I=12, r=3)
    Y, _ = L.mlp_fwd(X, gate, up, down, act)
    phi = {"swiglu": lambda x: x * special.expit(x),
           "geglu_tanh": lambda x: 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x**3)))}[act]

    def merged(p):
        return p["W"] + p["s"] * (p["A"] @ p["B"])

    ref = (phi(X @ merged(gate)) * (X @ merged(up))) @ merged(down)
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_B_zero_gives_base_output_and_zero_dA():
    X, dY, gate, up, down = _mlp_problem(seed=4, zero_B=True)
    Y, saved = L.mlp_fwd(X, gate, up, down)
    base = (X @ gate["W"]) * special.expit(X @ gate["W"]) * (X @ up["W"]) @ down["W"]
    assert np.array_equal(Y, base) or np.abs(Y - base).max() <= 1e-14 * np.abs(base).max()
    g = L.mlp_bwd(dY, X, saved, gate, up, down)
    for n in ("dA_g", "dA_u", "dA_d"):
        assert np.all(g[n] == 0), n


def test_A_zero_gives_zero_dB_and_s_zero_gives_zero_adapter_grads():
    X, dY, gate, up, down = _mlp_problem(seed=5, zero_A=True)
    Y, saved = L.mlp_fwd(X, gate, up, down)
    g = L.mlp_bwd(dY, X, saved, gate, up, down)
    for n in ("dB_g", "dB_u", "dB_d"):
        assert np.all(g[n] == 0), n
    X, dY, gate, up, down = _mlp_problem(seed=6)
    for p in (gate, up, down):
        p["s"] = 0.0
    Y, saved = L.mlp_fwd(X, gate, up, down)
    base = (X @ gate["W"]) * special.expit(X @ gate["W"]) * (X @ up["W"]) @ down["W"]
    np.testing.assert_allclose(Y, base, rtol=0, atol=1e-14 * np.abs(base).max())
    g = L.mlp_bwd(dY, X, saved, gate, up, down)
    for n in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        assert np.all(g[n] == 0), n


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_hoisted_product_is_bitwise_identical(dtype):
    """The commit that hoists dY @ B.t() states the results are bitwise
    identical; the oracle's hoisted and recomputed forms must agree exactly."""
    X, dY, gate, up, down = _mlp_problem(seed=7, T=64, H=32, I=48, r=4)
    X, dY = X.astype(dtype), dY.astype(dtype)
    gate, up, down = (L.as_dtype(p, dtype) for p in (gate, up, down))
    Y, saved = L.mlp_fwd(X, gate, up, down)
    a = L.mlp_bwd(dY, X, saved, gate, up, down, hoist=True)
    b = L.mlp_bwd(dY, X, saved, gate, up, down, hoist=False)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_token_permutation_permutes_rows():
    X, dY, gate, up, down = _mlp_problem(seed=8, T=9)
    perm = np.random.default_rng(0).permutation(X.shape[0])
    Y, saved = L.mlp_fwd(X, gate, up, down)
    g = L.mlp_bwd(dY, X, saved, gate, up, down)
    Yp, savedp = L.mlp_fwd(X[perm], gate, up, down)
    gp = L.mlp_bwd(dY[perm], X[perm], savedp, gate, up, down)
    np.testing.assert_allclose(Yp, Y[perm], rtol=0, atol=1e-14 * np.abs(Y).max())
    np.testing.assert_allclose(gp["dX"], g["dX"][perm], rtol=0, atol=1e-14 * np.abs(g["dX"]).max())
    for k in ("dA_g", "dB_g", "dA_u", "dB_u", "dA_d", "dB_d"):
        np.testing.assert_allclose(gp[k], g[k], rtol=0, atol=1e-12 * np.abs(g[k]).max())


def test_qkv_equals_three_single_projections():
    rng = np.random.default_rng(9)
    T, H, r = 6, 16, 4
    X = rng.standard_normal((T, H))
    q, k, v = _proj(rng, H, 16, r, 2.0), _proj(rng, H, 8, r, 2.0), _proj(rng, H, 8, r, 2.0)
    dQ, dK, dV = (rng.standard_normal((T, n)) for n in (16, 8, 8))
    (Q, K, V), saved = L.qkv_fwd(X, q, k, v)
    g = L.qkv_bwd(dQ, dK, dV, X, saved, q, k, v)
    dX = 0
    for out, dout, p, n in ((Q, dQ, q, "q"), (K, dK, k, "k"), (V, dV, v, "v")):
        Z = X @ p["W"] + p["s"] * (X @ p["A"]) @ p["B"]
        np.testing.assert_allclose(out, Z, rtol=0, atol=1e-13)
        gd = L.o_bwd(dout, X, dict(U=X @ p["A"]), p)
        dX = dX + gd["dX"]
        np.testing.assert_allclose(g["dA_" + n], gd["dA"], rtol=0, atol=1e-13)
        np.testing.assert_allclose(g["dB_" + n], gd["dB"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["dX"], dX, rtol=0, atol=1e-12)


def test_activation_special_values():
    x0 = np.zeros(1)
    for phi, dphi in L.ACTIVATIONS.values():
        assert phi(x0)[0] == 0.0
        assert abs(dphi(x0)[0] - 0.5) < 1e-15
        big = np.array([100.0, 40.0])
        assert np.allclose(phi(big) / big, 1.0, atol=1e-12)
        assert np.allclose(dphi(big), 1.0, atol=1e-12)
        neg = np.array([-100.0, -40.0])
        assert np.all(np.abs(phi(neg)) < 1e-12) and np.all(np.isfinite(dphi(neg)))
        for dt in (np.float32, np.float64):
            xx = np.array([-100, -20, 0, 20, 100], dtype=dt)
            assert np.all(np.isfinite(phi(xx))) and np.all(np.isfinite(dphi(xx)))
    # SiLU against the logistic function of scipy; GELU-tanh within 1e-3 of the
    # exact GELU x * Phi(x).
    x = np.linspace(-8, 8, 2001)
    np.testing.assert_allclose(L.silu(x), x * special.expit(x), rtol=1e-14, atol=1e-15)
    # the tanh form stays within 4.8e-4 of the exact GELU (its largest gap, near |x| = 2)
    assert np.abs(L.gelu_tanh(x) - x * special.ndtr(x)).max() < 5e-4
    # derivatives against central differences of the scalar functions
    for phi, dphi in L.ACTIVATIONS.values():
        h = 1e-6
        np.testing.assert_allclose(dphi(x), (phi(x + h) - phi(x - h)) / (2 * h), rtol=0, atol=1e-8)


def test_adapter_parameter_count_matches_page(golden_dir):
    """Adapters are A [in, r] and B [r, out]: r * (in + out) per projection.
    The Axolotl page states the total for Qwen3-8B at rank 16."""
    import os

    with open(os.path.join(golden_dir, "qwen3_8b_rank16_adapter_params.txt")) as f:
        line = [ln for ln in f if not ln.startswith("#")][0].split()
    total, layers, hidden, inter, nq, nkv, hd, r = map(int, line)
    shapes = [(hidden, nq * hd), (hidden, nkv * hd), (hidden, nkv * hd), (nq * hd, hidden),
              (hidden, inter), (hidden, inter), (inter, hidden)]
    # the oracle's projection takes A [in, r] and B [r, out] (checked on a
    # scaled-down copy of each shape), so a projection has r * (in + out)
    per_layer = 0
    for n_in, n_out in shapes:
        a, b = n_in // 128, n_out // 128
        A = np.zeros((a, r), np.float32)
        B = np.zeros((r, b), np.float32)
        Z, U = L.proj_fwd(np.ones((2, a), np.float32), np.ones((a, b), np.float32), A, B, 2.0)
        assert Z.shape == (2, b) and U.shape == (2, r)
        per_layer += r * (n_in + n_out)
    assert per_layer * layers == total


def test_fp32_lora_mode_matches_integer_brute_force():
    """fp32 LoRA-gradient mode ("LoRA Optimizations", section "FP32 LoRA
    gradients"): the adapters are rounded to bf16 before the products and the
    gradients come out in fp32 without a final rounding.  With small integer
    inputs and adapters of the form a * (1 + 2^-10) (which round to the
    integer a), every product and sum is an exact integer, so the mode's
    gradients must equal Python-integer brute force over the rounded
    adapters exactly, and must hold values that a bf16 result could not."""
    rng = np.random.default_rng(5)
    T, K, N, r, s = 300, 12, 10, 3, 2.0

    def ints(shape, p):
        return (rng.integers(-3, 4, shape) * (rng.random(shape) < p)).astype(np.float32)

    X, dY = ints((T, K), 0.8), ints((T, N), 0.8)
    A_int, B_int = ints((K, r), 0.7), ints((r, N), 0.7)
    W = rng.standard_normal((K, N)).astype(np.float32)
    bump = np.float32(1 + 2.0 ** -10)
    o = dict(W=W, A=A_int * bump, B=B_int * bump, s=s)
    assert not np.array_equal(o["A"], A_int)  # the fp32 adapters are not integers
    oc = L.to_compute_adapters(o)
    assert np.array_equal(oc["A"], A_int) and np.array_equal(oc["B"], B_int)
    Y, saved = L.o_fwd(X, oc)
    got = L.o_bwd(dY, X, saved, oc)
    assert got["dA"].dtype == np.float32 and got["dB"].dtype == np.float32

    Xi, dYi = X.astype(int).tolist(), dY.astype(int).tolist()
    Ai, Bi = A_int.astype(int).tolist(), B_int.astype(int).tolist()
    U = [[sum(Xi[t][k] * Ai[k][i] for k in range(K)) for i in range(r)] for t in range(T)]
    P = [[sum(dYi[t][n] * Bi[i][n] for n in range(N)) for i in range(r)] for t in range(T)]
    dA = [[2 * sum(Xi[t][k] * P[t][i] for t in range(T)) for i in range(r)] for k in range(K)]
    dB = [[2 * sum(U[t][i] * dYi[t][n] for t in range(T)) for n in range(N)] for i in range(r)]
    assert np.array_equal(got["dA"], np.array(dA, np.float32))
    assert np.array_equal(got["dB"], np.array(dB, np.float32))
    # sharp: rounding these gradients to bf16 would change some of them
    from oracle.nf4 import round_to_bf16

    for g in (got["dA"], got["dB"]):
        assert np.any(round_to_bf16(g) != g)


def _relu2_problem(seed=6, T=4, H=8, I=12, r=2):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, H))
    dY = rng.standard_normal((T, H))
    up = _proj(rng, H, I, r, 1.25)
    down = _proj(rng, I, H, r, 2.0)
    return X, dY, up, down


def test_relu2_mlp_gradients_match_finite_differences():
    X, dY, up, down = _relu2_problem()
    Y, saved = L.relu2_mlp_fwd(X, up, down)
    assert np.abs(saved["u"]).min() > 1e-3  # away from the kink of 2 max(u, 0) at 0
    assert (saved["u"] > 0).any() and (saved["u"] < 0).any()

    def loss():
        Yv, _ = L.relu2_mlp_fwd(X, up, down)
        return float(np.sum(Yv * dY))

    g = L.relu2_mlp_bwd(dY, X, saved, up, down)
    _assert_grad(g["dX"], _central_fd(loss, X), "dX")
    for name, p in (("u", up), ("d", down)):
        _assert_grad(g["dA_" + name], _central_fd(loss, p["A"]), "dA_" + name)
        _assert_grad(g["dB_" + name], _central_fd(loss, p["B"]), "dB_" + name)


def test_relu2_mlp_equals_base_mlp_on_merged_weights_and_special_values():
    X, dY, up, down = _relu2_problem(seed=7, T=5, H=8, I=12, r=3)
    Y, _ = L.relu2_mlp_fwd(X, up, down)

    def merged(p):
        return p["W"] + p["s"] * (p["A"] @ p["B"])

    pre = X @ merged(up)
    ref = np.where(pre > 0, pre * pre, 0.0) @ merged(down)
    np.testing.assert_allclose(Y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    x = np.array([-2.0, -1e-300, 0.0, 0.5, 3.0])
    assert np.array_equal(L.relu2(x), [0.0, 0.0, 0.0, 0.25, 9.0])
    assert np.array_equal(L.relu2_grad(x), [0.0, 0.0, 0.0, 1.0, 6.0])
    # B = 0 on both projections: the base ReLU^2 MLP and zero dA
    up0, down0 = dict(up, B=np.zeros_like(up["B"])), dict(down, B=np.zeros_like(down["B"]))
    Y0, s0 = L.relu2_mlp_fwd(X, up0, down0)
    base = np.where(X @ up["W"] > 0, (X @ up["W"]) ** 2, 0.0) @ down["W"]
    np.testing.assert_allclose(Y0, base, rtol=0, atol=1e-12 * np.abs(base).max())
    g0 = L.relu2_mlp_bwd(dY, X, s0, up0, down0)
    assert not g0["dA_u"].any() and not g0["dA_d"].any()


def test_activations_match_pytorch_implementations():
    """phi and phi' against PyTorch's own float64 SiLU and tanh-form GELU
    (torch.nn.functional.silu, gelu(approximate="tanh")), derivatives by
    autograd: an implementation independent of the oracle's, so a slip in a
    constant (0.044715, sqrt(2/pi)) or in a derivative term fails here."""
    import torch
    import torch.nn.functional as F

    xs = np.concatenate([np.linspace(-12, 12, 4801), [-1e-3, 1e-3, 0.5, 1.0, 2.0, 3.0]])
    for phi, dphi, ref in ((L.silu, L.silu_grad, F.silu),
                           (L.gelu_tanh, L.gelu_tanh_grad, lambda t: F.gelu(t, approximate="tanh"))):
        x = torch.tensor(xs, dtype=torch.float64, requires_grad=True)
        y = ref(x)
        (dy,) = torch.autograd.grad(y.sum(), x)
        np.testing.assert_allclose(phi(xs), y.detach().numpy(), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(dphi(xs), dy.numpy(), rtol=1e-12, atol=1e-14)
