"""GPU parity of the HIP path against the CPU oracle on the same seeded inputs.

Shapes here span several 256-row / 256-column tiles with ragged tails and
run in seconds on the oracle, up to operands at the kernels' 2 GiB limit;
the benchmark shapes are in test_gpu_configs.py.  Bar: max|err|/max|ref| <= 2e-2 per output tensor in
bf16 (fp32 accumulation), <= 1e-5 in fp32; NF4 codes and dequantized weights
bit-exact.
"""
import numpy as np
import pytest

from oracle import lora as OL
from oracle import nf4 as ON
from workload import WorkloadConfig, make_attn_inputs, make_mlp_inputs, make_relu2_inputs
from _util import TOL, assert_close, dev, host, proj_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lm():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import adapter_mlp_amd

    adapter_mlp_amd.load()
    return adapter_mlp_amd


def _mlp_case(lm, cfg, act, seed=None):
    """Forward + backward of one gated MLP against the oracle.  With cfg.nf4
    the three bases are NF4-quantized on the GPU (checked bit for bit against
    the oracle quantizer) and the oracle runs on the dequantized weights; with
    cfg.lora_dtype == "f32" the adapters are fp32 and the oracle multiplies
    with them as the mode casts them."""
    import torch

    inp = make_mlp_inputs(cfg, seed=seed)
    dt = cfg.dtype
    tol = TOL[dt]
    nf = {}
    if cfg.nf4:
        for k in ("gate", "up", "down"):
            nf[k] = _nf4_dev(lm, inp[k]["W"])
            q = _check_nf4_bitexact(lm, inp[k]["W"], nf[k])
            inp[k] = dict(inp[k], W=ON.dequantize(q, "bf16"))
    ad = cfg.lora_dtype or None
    X, dY = dev(inp["X"], dt), dev(inp["dY"], dt)
    g, u, d = (proj_dev(inp[k], dt, nf4=nf.get(k), adapters=ad) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, act)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, act)
    torch.cuda.synchronize()
    if ad:
        assert all(t.dtype == torch.float32 for t in grads.values())
        inp = dict(inp, **{k: OL.to_compute_adapters(inp[k]) for k in ("gate", "up", "down")})
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], act)
    assert_close("Y", host(Y), Yr, tol)
    assert_close("e", host(saved["e"]), sr["e"], tol)
    assert_close("g", host(saved["g"]), sr["g"], tol)
    r = cfg.r
    Ur = np.concatenate([sr["U_g"], sr["U_u"], sr["U_d"]], axis=1)
    assert_close("U", host(saved["U"]), Ur, tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
                         ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)
    return Y, dX, grads


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_mlp_bf16_ragged(lm, act):
    cfg = WorkloadConfig(90, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act=act)
    _mlp_case(lm, cfg, act)


def test_mlp_bf16_rank32(lm):
    # r = 32 (2r = 64, the widest gate/up adapter group): the dg / de rank-r
    # passes do not fuse and run one after the other on shared scratch
    cfg = WorkloadConfig(89, "mlp", T=300, H=512, I=1088, r=32, alpha=16, dtype="bf16", act="swiglu")
    _mlp_case(lm, cfg, "swiglu")


def test_mlp_bf16_rank24(lm):
    # a rank that is not a multiple of 16: partial 16-column blocks in the
    # unfused rank-r products
    cfg = WorkloadConfig(88, "mlp", T=200, H=256, I=640, r=24, alpha=24, dtype="bf16", act="geglu_tanh")
    _mlp_case(lm, cfg, "geglu_tanh")


def test_mlp_bf16_rank8_scale_not_power_of_two(lm):
    cfg = WorkloadConfig(91, "mlp", T=200, H=256, I=640, r=8, alpha=12, dtype="bf16", act="swiglu")
    _mlp_case(lm, cfg, "swiglu")


def test_mlp_fp32_tiny_config(lm):
    from workload import CONFIGS

    _mlp_case(lm, CONFIGS[1], "swiglu")


def test_mlp_fp32_odd_shapes(lm):
    cfg = WorkloadConfig(92, "mlp", T=37, H=72, I=100, r=3, alpha=5, dtype="f32", act="geglu_tanh",
                         rms_inputs=False)
    _mlp_case(lm, cfg, "geglu_tanh")


def _qkv_case(lm, cfg):
    """Q/K/V and O forward + backward against the oracle.  With cfg.nf4 every
    base (q, k, v, o) is NF4-quantized on the GPU, checked bit for bit, and
    the oracle runs on the dequantized weights; cfg.lora_dtype == "f32" selects
    fp32 adapters (the oracle takes them as the mode casts them)."""
    import torch

    inp = make_attn_inputs(cfg)
    dt = cfg.dtype
    tol = TOL[dt]
    nf = {}
    if cfg.nf4:
        for n in ("q", "k", "v", "o"):
            nf[n] = _nf4_dev(lm, inp[n]["W"])
            qz = _check_nf4_bitexact(lm, inp[n]["W"], nf[n])
            inp[n] = dict(inp[n], W=ON.dequantize(qz, "bf16"))
    ad = cfg.lora_dtype or None
    X = dev(inp["X"], dt)
    q, k, v = (proj_dev(inp[n], dt, nf4=nf.get(n), adapters=ad) for n in ("q", "k", "v"))
    Q, K, V, U = lm.qkv_fwd(X, q, k, v)
    dQ, dK, dV = (dev(inp[n], dt) for n in ("dQ", "dK", "dV"))
    dX, grads = lm.qkv_bwd(dQ, dK, dV, X, U, q, k, v)
    Xo = dev(inp["Xo"], dt)
    o = proj_dev(inp["o"], dt, nf4=nf.get("o"), adapters=ad)
    Yo, Uo = lm.o_fwd(Xo, o)
    dXo, dAo, dBo = lm.o_bwd(dev(inp["dO"], dt), Xo, Uo, o)
    torch.cuda.synchronize()
    if ad:
        assert all(t.dtype == torch.float32 for t in list(grads.values()) + [dAo, dBo])
        inp = dict(inp, **{n: OL.to_compute_adapters(inp[n]) for n in ("q", "k", "v", "o")})
    (Qr, Kr, Vr), sr = OL.qkv_fwd(inp["X"], inp["q"], inp["k"], inp["v"])
    gr = OL.qkv_bwd(inp["dQ"], inp["dK"], inp["dV"], inp["X"], sr, inp["q"], inp["k"], inp["v"])
    for name, a, b in (("Q", Q, Qr), ("K", K, Kr), ("V", V, Vr)):
        assert_close(name, host(a), b, tol)
    assert_close("U", host(U), np.concatenate([sr["U_q"], sr["U_k"], sr["U_v"]], axis=1), tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for n in ("dA_q", "dB_q", "dA_k", "dB_k", "dA_v", "dB_v"):
        assert_close(n, host(grads[n]), gr[n], tol)
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    go = OL.o_bwd(inp["dO"], inp["Xo"], so, inp["o"])
    assert_close("O", host(Yo), Yr, tol)
    assert_close("dX_o", host(dXo), go["dX"], tol)
    assert_close("dA_o", host(dAo), go["dA"], tol)
    assert_close("dB_o", host(dBo), go["dB"], tol)


@pytest.mark.parametrize("r", [8, 16])
def test_qkv_o_bf16_ragged(lm, r):
    cfg = WorkloadConfig(93, "attn", T=300, H=512, r=r, alpha=32, dtype="bf16", Nq=512, Nk=192, Nv=128)
    _qkv_case(lm, cfg)


@pytest.mark.parametrize("T", [0, 1, 257])
def test_qkv_o_edge_token_counts(lm, T):
    # one token, a ragged 257, and T = 0, which must still overwrite every
    # adapter gradient with zeros (the three rank-r passes run batched)
    import torch

    cfg = WorkloadConfig(92, "attn", T=T, H=256, r=16, alpha=32, dtype="bf16", Nq=256, Nk=128, Nv=64)
    if T > 0:
        _qkv_case(lm, cfg)
        return
    inp = make_attn_inputs(cfg)
    X = dev(inp["X"])
    q, k, v = (proj_dev(inp[n]) for n in ("q", "k", "v"))
    Q, K, V, U = lm.qkv_fwd(X, q, k, v)
    grads = {f"d{ab}_{n}": torch.full_like(getattr(p, ab), 7.0) for n, p in (("q", q), ("k", k), ("v", v))
             for ab in ("A", "B")}
    dX, grads = lm.qkv_bwd(*(dev(inp[n]) for n in ("dQ", "dK", "dV")), X, U, q, k, v, grads=grads)
    o = proj_dev(inp["o"])
    Xo = dev(inp["Xo"])
    Yo, Uo = lm.o_fwd(Xo, o)
    dA, dB = torch.full_like(o.A, 7.0), torch.full_like(o.B, 7.0)
    lm.o_bwd(dev(inp["dO"]), Xo, Uo, o, dA=dA, dB=dB)
    torch.cuda.synchronize()
    for name, t in list(grads.items()) + [("dA_o", dA), ("dB_o", dB)]:
        assert torch.all(t == 0), name


@pytest.mark.parametrize("r", [40, 64])
def test_o_bf16_wide_rank(lm, r):
    # the single projection takes ranks up to 64 (three and four 16-column blocks)
    import torch

    cfg = WorkloadConfig(91, "attn", T=300, H=512, r=r, alpha=32, dtype="bf16", Nq=384, Nk=64, Nv=64)
    inp = make_attn_inputs(cfg)
    Xo = dev(inp["Xo"])
    o = proj_dev(inp["o"])
    Yo, Uo = lm.o_fwd(Xo, o)
    dXo, dAo, dBo = lm.o_bwd(dev(inp["dO"]), Xo, Uo, o)
    torch.cuda.synchronize()
    Yr, so = OL.o_fwd(inp["Xo"], inp["o"])
    go = OL.o_bwd(inp["dO"], inp["Xo"], so, inp["o"])
    tol = TOL["bf16"]
    assert_close("O", host(Yo), Yr, tol)
    assert_close("U_o", host(Uo), so["U"], tol)
    assert_close("dX_o", host(dXo), go["dX"], tol)
    assert_close("dA_o", host(dAo), go["dA"], tol)
    assert_close("dB_o", host(dBo), go["dB"], tol)


def test_qkv_o_fp32(lm):
    cfg = WorkloadConfig(94, "attn", T=50, H=96, r=4, alpha=8, dtype="f32", Nq=96, Nk=32, Nv=40)
    _qkv_case(lm, cfg)


# QLoRA on the attention projections ("loralei" README, section "Use": the
# QLoRA example quantizes q, k, v and o).  The Q/K/V forward walks three NF4
# regions across N (a ragged 192- and 128-column region after the first), the
# Q/K/V input gradient three NF4 K segments, and O one NF4 weight each way.
@pytest.mark.parametrize("T", [1, 257, 300])
def test_qkv_o_nf4_base(lm, T):
    cfg = WorkloadConfig(103, "attn", T=T, H=512, r=16, alpha=32, dtype="bf16", Nq=512, Nk=192, Nv=128, nf4=True)
    _qkv_case(lm, cfg)


def test_qkv_o_nf4_base_fp32_adapters(lm):
    cfg = WorkloadConfig(104, "attn", T=300, H=512, r=16, alpha=32, dtype="bf16", Nq=512, Nk=192, Nv=128, nf4=True,
                         lora_dtype="f32")
    _qkv_case(lm, cfg)


# ---------------------------------------------------------------------------
# Ungated ReLU^2 MLP
# ---------------------------------------------------------------------------

def _relu2_case(lm, cfg, nf4=False):
    import torch

    inp = make_relu2_inputs(cfg)
    dt = cfg.dtype
    nf = {}
    if nf4:
        for k in ("up", "down"):
            w = lm.nf4_quantize(dev(inp[k]["W"]))
            q = ON.quantize(inp[k]["W"])
            torch.cuda.synchronize()
            assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), f"{k}: NF4 codes differ"
            nf[k] = w
            inp[k] = dict(inp[k], W=ON.dequantize(q, "bf16"))
    ad = cfg.lora_dtype or None
    X, dY = dev(inp["X"], dt), dev(inp["dY"], dt)
    up, down = (proj_dev(inp[k], dt, nf4=nf.get(k), adapters=ad) for k in ("up", "down"))
    Y, saved = lm.relu2_mlp_fwd(X, up, down)
    dX, grads = lm.relu2_mlp_bwd(dY, X, saved, up, down)
    torch.cuda.synchronize()
    if ad:
        assert all(t.dtype == torch.float32 for t in grads.values())
        inp = dict(inp, up=OL.to_compute_adapters(inp["up"]), down=OL.to_compute_adapters(inp["down"]))
    Yr, sr = OL.relu2_mlp_fwd(inp["X"], inp["up"], inp["down"])
    gr = OL.relu2_mlp_bwd(inp["dY"], inp["X"], sr, inp["up"], inp["down"])
    tol = TOL[dt]
    assert_close("Y", host(Y), Yr, tol)
    assert_close("u", host(saved["u"]), sr["u"], tol)
    assert_close("U", host(saved["U"]), np.concatenate([sr["U_u"], sr["U_d"]], axis=1), tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in (("dA_up", "dA_u"), ("dB_up", "dB_u"), ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)
    return Y, dX, grads


def test_relu2_mlp_bf16_ragged(lm):
    cfg = WorkloadConfig(97, "relu2", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16")
    _relu2_case(lm, cfg)


@pytest.mark.slow
def test_relu2_mlp_bf16_maximum_extent(lm):
    # u, h and du of T x I bf16 just under 2 GiB (T = 65535, a 255-row tail);
    # the oracle runs on row chunks and the adapter gradients, sums over
    # tokens, are added in fp64 over the chunks
    import torch

    T, H, I = 65535, 64, 16384
    cfg = WorkloadConfig(93, "relu2", T=T, H=H, I=I, r=16, alpha=32, dtype="bf16")
    inp = make_relu2_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    up, down = (proj_dev(inp[k]) for k in ("up", "down"))
    Y, saved = lm.relu2_mlp_fwd(X, up, down)
    dX, grads = lm.relu2_mlp_bwd(dY, X, saved, up, down)
    torch.cuda.synchronize()
    gkeys = (("dA_up", "dA_u"), ("dB_up", "dB_u"), ("dA_down", "dA_d"), ("dB_down", "dB_d"))
    Yr, dXr = np.zeros((T, H)), np.zeros((T, H))
    sums = {k: 0.0 for _, k in gkeys}
    u_err, u_ref = 0.0, 0.0
    CH = 8192
    for t0 in range(0, T, CH):
        sl = slice(t0, min(T, t0 + CH))
        Yc, sc = OL.relu2_mlp_fwd(inp["X"][sl], inp["up"], inp["down"])
        gc = OL.relu2_mlp_bwd(inp["dY"][sl], inp["X"][sl], sc, inp["up"], inp["down"])
        Yr[sl], dXr[sl] = Yc, gc["dX"]
        for _, k in gkeys:
            sums[k] = sums[k] + gc[k].astype(np.float64)
        got = host(saved["u"][sl])
        assert np.all(np.isfinite(got)), f"u: non-finite values in rows {t0}.."
        u_err = max(u_err, float(np.abs(got - sc["u"]).max()))
        u_ref = max(u_ref, float(np.abs(sc["u"]).max()))
    tol = TOL["bf16"]
    print(f"  u        max|err|/max|ref| = {u_err / u_ref:.3e} (tol {tol:g})", flush=True)
    assert u_err <= tol * u_ref
    assert_close("Y", host(Y), Yr, tol)
    assert_close("dX", host(dX), dXr, tol)
    for k_dev, k_ref in gkeys:
        assert_close(k_dev, host(grads[k_dev]), sums[k_ref], tol)


def test_relu2_mlp_bf16_rank64(lm):
    # the widest adapter: four 16-column blocks in every rank-r product
    cfg = WorkloadConfig(87, "relu2", T=260, H=256, I=512, r=64, alpha=64, dtype="bf16")
    _relu2_case(lm, cfg)


def test_relu2_mlp_bf16_rank32(lm):
    cfg = WorkloadConfig(98, "relu2", T=200, H=256, I=640, r=32, alpha=16, dtype="bf16")
    _relu2_case(lm, cfg)


def test_relu2_mlp_fp32_odd_shapes(lm):
    cfg = WorkloadConfig(99, "relu2", T=37, H=72, I=100, r=3, alpha=5, dtype="f32", rms_inputs=False)
    _relu2_case(lm, cfg)


def test_relu2_mlp_nf4_base(lm):
    cfg = WorkloadConfig(100, "relu2", T=260, H=256, I=512, r=16, alpha=32, dtype="bf16", nf4=True)
    _relu2_case(lm, cfg, nf4=True)


def test_relu2_mlp_fp32_lora_mode(lm):
    cfg = WorkloadConfig(101, "relu2", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", lora_dtype="f32")
    _relu2_case(lm, cfg)


@pytest.mark.parametrize("T", [0, 1, 257])
def test_relu2_mlp_edge_token_counts(lm, T):
    import torch

    cfg = WorkloadConfig(102, "relu2", T=T, H=256, I=512, r=16, alpha=32, dtype="bf16")
    if T > 0:
        _relu2_case(lm, cfg)
        return
    inp = make_relu2_inputs(cfg)
    X = torch.empty((0, cfg.H), dtype=torch.bfloat16, device="cuda:0")
    up, down = (proj_dev(inp[k]) for k in ("up", "down"))
    Y, saved = lm.relu2_mlp_fwd(X, up, down)
    grads = {k: torch.full_like(v, 7.0) for k, v in (("dA_up", up.A), ("dB_up", up.B), ("dA_down", down.A),
                                                      ("dB_down", down.B))}
    dX, grads = lm.relu2_mlp_bwd(X, X, saved, up, down, grads=grads)
    torch.cuda.synchronize()
    assert Y.shape == (0, cfg.H) and dX.shape == (0, cfg.H)
    for k, v in grads.items():
        assert not v.any(), f"{k} not zero-filled at T = 0"


# ---------------------------------------------------------------------------
# fp32 LoRA-gradient mode: bf16 inputs, fp32 adapters and adapter gradients
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
@pytest.mark.parametrize("r", [16, 32])
def test_fp32_lora_mode_mlp(lm, act, r):
    """Against the oracle fed the adapters as the mode casts them (bf16), and
    against the bf16 mode on the same casts: the forward outputs must agree
    bit for bit and the mode's fp32 gradients must round to the bf16 mode's."""
    import torch

    cfg = WorkloadConfig(95, "mlp", T=300, H=512, I=1088, r=r, alpha=32, dtype="bf16", act=act,
                         lora_dtype="f32")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k], adapters="f32") for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, act)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, act)
    cast = {k: OL.to_compute_adapters(inp[k]) for k in ("gate", "up", "down")}
    g16, u16, d16 = (proj_dev(cast[k]) for k in ("gate", "up", "down"))
    Y16, saved16 = lm.mlp_fwd(X, g16, u16, d16, act)
    dX16, grads16 = lm.mlp_bwd(dY, X, saved16, g16, u16, d16, act)
    torch.cuda.synchronize()
    assert all(t.dtype == torch.float32 for t in grads.values())
    Yr, sr = OL.mlp_fwd(inp["X"], cast["gate"], cast["up"], cast["down"], act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, cast["gate"], cast["up"], cast["down"], act)
    tol = TOL["bf16"]
    assert_close("Y", host(Y), Yr, tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
                         ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)
        assert torch.equal(grads[k_dev].to(torch.bfloat16), grads16[k_dev]), k_dev
    for a, b in ((Y, Y16), (saved["e"], saved16["e"]), (saved["g"], saved16["g"]), (saved["U"], saved16["U"]),
                 (dX, dX16)):
        assert torch.equal(a, b)


def _small_ints(rng, shape, p_nonzero, bump=1.0):
    """Values in {-1, 0, 1} (nonzero with probability p_nonzero), times bump."""
    v = rng.integers(0, 2, shape) * 2 - 1
    return (v * (rng.random(shape) < p_nonzero) * bump).astype(np.float32)


def test_fp32_lora_mode_qkv_o_gradients_exact(lm):
    """Inputs in {-1, 0, 1} and adapters a * (1 + 2^-10) that the mode's cast
    rounds to a: every rank-r intermediate is a small integer (exact in bf16)
    and every gradient an integer below 2^24 (exact in fp32 in any order), so
    the mode's fp32 dA and dB must equal the oracle's bit for bit.  Many of
    them are not bf16 values, so a rounded gradient would fail."""
    import torch

    rng = np.random.default_rng(96)
    T, H, Ns, r, s = 1000, 256, (256, 128, 64), 16, 2.0
    bump = np.float32(1 + 2.0 ** -10)

    def proj(n_in, n_out):
        W = ON.round_to_bf16((rng.standard_normal((n_in, n_out)) / 16).astype(np.float32))
        return dict(W=W, A=_small_ints(rng, (n_in, r), 0.25, bump), B=_small_ints(rng, (r, n_out), 0.25, bump), s=s)

    X = _small_ints(rng, (T, H), 0.5)
    q, k, v = (proj(H, n) for n in Ns)
    dZ = [_small_ints(rng, (T, n), 0.5) for n in Ns]
    o = proj(Ns[0], H)
    Xo, dO = _small_ints(rng, (T, Ns[0]), 0.5), _small_ints(rng, (T, H), 0.5)

    Xd = dev(X)
    qd, kd, vd, od = (proj_dev(p, adapters="f32") for p in (q, k, v, o))
    _, _, _, U = lm.qkv_fwd(Xd, qd, kd, vd)
    _, grads = lm.qkv_bwd(*(dev(z) for z in dZ), Xd, U, qd, kd, vd)
    Xod = dev(Xo)
    _, Uo = lm.o_fwd(Xod, od)
    _, dAo, dBo = lm.o_bwd(dev(dO), Xod, Uo, od)
    torch.cuda.synchronize()

    qc, kc, vc, oc = (OL.to_compute_adapters(p) for p in (q, k, v, o))
    _, sr = OL.qkv_fwd(X, qc, kc, vc)
    assert max(np.abs(sr[n]).max() for n in ("U_q", "U_k", "U_v")) <= 256  # exact in bf16
    gr = OL.qkv_bwd(*dZ, X, sr, qc, kc, vc)
    _, so = OL.o_fwd(Xo, oc)
    gor = OL.o_bwd(dO, Xo, so, oc)
    got = {n: host(grads[n]) for n in grads}
    got.update(dA_o=host(dAo), dB_o=host(dBo))
    ref = {n: gr[n] for n in grads}
    ref.update(dA_o=gor["dA"], dB_o=gor["dB"])
    for n in got:
        assert np.abs(ref[n]).max() < 2 ** 24
        assert np.array_equal(got[n], ref[n]), f"{n}: {np.abs(got[n] - ref[n]).max()}"
    assert any(np.any(ON.round_to_bf16(ref[n]) != ref[n]) for n in ref)


# ---------------------------------------------------------------------------
# NF4
# ---------------------------------------------------------------------------

def _nf4_dev(lm, W32):
    import torch

    w = lm.nf4_quantize(dev(W32, "bf16"))
    torch.cuda.synchronize()
    return w


def _check_nf4_bitexact(lm, W32, w):
    q = ON.quantize(W32)
    assert np.array_equal(w.codes.cpu().numpy(), q["codes"]), "packed codes differ"
    assert np.array_equal(w.q8.cpu().numpy(), q["q8"]), "q8 differ"
    assert np.array_equal(w.s2.cpu().numpy().view(np.uint32), q["s2"].view(np.uint32)), "s2 differ"
    assert w.mu.cpu().numpy().view(np.uint32)[0] == np.float32(q["mu"]).view(np.uint32), "mu differs"
    return q


def test_nf4_quantize_dequant_unpack_bitexact(lm):
    import torch

    rng = np.random.default_rng(95)
    W = ON.round_to_bf16((rng.standard_normal((512, 256)) / 16).astype(np.float32))
    W[3, :64] = 0.0  # an all-zero block
    w = _nf4_dev(lm, W)
    q = _check_nf4_bitexact(lm, W, w)
    codes = lm.nf4_unpack_codes(w)
    d32 = lm.nf4_dequant(w, torch.float32)
    d16 = lm.nf4_dequant(w, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), ON.unpack_codes(q["codes"]))
    assert np.array_equal(d32.cpu().numpy().view(np.uint32), ON.dequantize(q, "f32").view(np.uint32))
    ref16 = ON.dequantize(q, "bf16")
    got16 = d16.view(torch.int16).cpu().numpy().astype(np.uint16).astype(np.uint32) << 16
    assert np.array_equal(got16, ref16.view(np.uint32))


def test_nf4_quantize_fp32_input_bitexact(lm):
    import torch

    rng = np.random.default_rng(96)
    W = (rng.standard_normal((128, 256)) * 0.05).astype(np.float32)
    w = lm.nf4_quantize(dev(W, "f32"))
    torch.cuda.synchronize()
    _check_nf4_bitexact(lm, W, w)


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
@pytest.mark.parametrize("r", [16, 32])
def test_qlora_mlp_bf16(lm, act, r):
    import torch

    cfg = WorkloadConfig(97, "mlp", T=300, H=512, I=1024, r=r, alpha=32, dtype="bf16", act=act, nf4=True)
    inp = make_mlp_inputs(cfg)
    nf4 = {k: _nf4_dev(lm, inp[k]["W"]) for k in ("gate", "up", "down")}
    for k in nf4:
        q = _check_nf4_bitexact(lm, inp[k]["W"], nf4[k])
        inp[k] = dict(inp[k], W=ON.dequantize(q, "bf16"))
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k], "bf16", nf4=nf4[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, act)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, act)
    torch.cuda.synchronize()
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"], act)
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"], act)
    assert_close("Y", host(Y), Yr, TOL["bf16"])
    assert_close("dX", host(dX), gr["dX"], TOL["bf16"])
    for k_dev, k_ref in (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
                         ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], TOL["bf16"])


# I = 1088 = 8 x 128 + 64: the last gate/up tile holds 64 gate and 64 up
# columns, so half of every NF4 column pair it unpacks lies past I.
@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_qlora_mlp_ragged_dual_tile(lm, act):
    cfg = WorkloadConfig(105, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act=act, nf4=True)
    _mlp_case(lm, cfg, act)


@pytest.mark.parametrize("act", ["swiglu", "geglu_tanh"])
def test_qlora_mlp_fp32_adapters(lm, act):
    cfg = WorkloadConfig(106, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act=act, nf4=True,
                         lora_dtype="f32")
    _mlp_case(lm, cfg, act)


# (rows, cols) of the NF4 weight: K = rows (forward) or cols (transposed) is
# 1, 2, 3 or more K steps of 64, and N leaves ragged tiles of 64 or 128.
@pytest.mark.parametrize("shape", [(512, 768), (64, 512), (128, 384), (192, 256)])
@pytest.mark.parametrize("trans", [False, True])
@pytest.mark.parametrize("with_lora", [False, True])
def test_nf4_gemm(lm, shape, trans, with_lora):
    import torch

    rng = np.random.default_rng(98)
    (rows, cols), T, r, s = shape, 300, 16, 2.0
    W = ON.round_to_bf16((rng.standard_normal((rows, cols)) / np.sqrt(rows)).astype(np.float32))
    A = ON.round_to_bf16(rng.uniform(-1, 1, (rows, r)).astype(np.float32) / np.sqrt(rows))
    B = ON.round_to_bf16((rng.standard_normal((r, cols)) * 0.02).astype(np.float32))
    X = ON.round_to_bf16(rng.standard_normal((T, cols if trans else rows)).astype(np.float32))
    w = _nf4_dev(lm, W)
    q = _check_nf4_bitexact(lm, W, w)
    Wd = ON.dequantize(q, "bf16")
    Y = lm.nf4_gemm(dev(X), w, dev(A) if with_lora else None, dev(B) if with_lora else None, s, trans)
    torch.cuda.synchronize()
    # the oracle's projection on the dequantized weight: its forward for
    # trans = 0, and for trans = 1 the input gradient of its backward with
    # dZ = X (Y = X deq(W)^T + s (X B^T) A^T); without adapters A = B = 0
    if not with_lora:
        A, B = np.zeros_like(A), np.zeros_like(B)
    if not trans:
        ref, _ = OL.proj_fwd(X, Wd, A, B, s)
    else:
        X_in, U = np.zeros((T, rows), np.float32), np.zeros((T, r), np.float32)
        ref, _, _ = OL.proj_bwd(X, X_in, Wd, A, B, s, U)
    assert_close("Y", host(Y), ref, TOL["bf16"])


# ---------------------------------------------------------------------------
# Edge cases and invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [0, 1, 255, 257])
def test_mlp_edge_token_counts(lm, T):
    import torch

    cfg = WorkloadConfig(99, "mlp", T=T, H=256, I=320, r=16, alpha=32, dtype="bf16")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d)
    grads = dict(dA_gate=torch.full_like(g.A, 7.0), dB_gate=torch.full_like(g.B, 7.0),
                 dA_up=torch.full_like(u.A, 7.0), dB_up=torch.full_like(u.B, 7.0),
                 dA_down=torch.full_like(d.A, 7.0), dB_down=torch.full_like(d.B, 7.0))
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, grads=grads)
    torch.cuda.synchronize()
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"])
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"])
    if T == 0:
        for kk, vv in grads.items():
            assert torch.all(vv == 0), kk  # outputs are overwritten, not accumulated
        return
    assert_close("Y", host(Y), Yr, TOL["bf16"])
    assert_close("dX", host(dX), gr["dX"], TOL["bf16"])
    assert_close("dA_gate", host(grads["dA_gate"]), gr["dA_g"], TOL["bf16"])
    assert_close("dB_down", host(grads["dB_down"]), gr["dB_d"], TOL["bf16"])


@pytest.mark.slow
def test_mlp_bf16_maximum_extent(lm):
    # The largest activation the kernels' 32-bit operand offsets accept: T x I
    # bf16 just under 2 GiB (T = 65535: 255 whole 256-row tiles and a 255-row
    # tail).  H = 64 keeps the oracle's products small; it runs on row chunks
    # (Y, e, g and dX rows are per token; every dA and dB is a sum over
    # tokens, added here in fp64 over the chunks).
    import torch

    T, H, I = 65535, 64, 16384
    cfg = WorkloadConfig(94, "mlp", T=T, H=H, I=I, r=16, alpha=32, dtype="bf16", act="swiglu")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d, "swiglu")
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, "swiglu")
    torch.cuda.synchronize()
    gkeys = (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
             ("dA_down", "dA_d"), ("dB_down", "dB_d"))
    Yr, dXr = np.zeros((T, H)), np.zeros((T, H))
    sums = {k: 0.0 for _, k in gkeys}
    err = {"e": [0.0, 0.0], "g": [0.0, 0.0]}  # max|err|, max|ref| over the chunks
    CH = 8192
    for t0 in range(0, T, CH):
        sl = slice(t0, min(T, t0 + CH))
        Yc, sc = OL.mlp_fwd(inp["X"][sl], inp["gate"], inp["up"], inp["down"], "swiglu")
        gc = OL.mlp_bwd(inp["dY"][sl], inp["X"][sl], sc, inp["gate"], inp["up"], inp["down"], "swiglu")
        Yr[sl], dXr[sl] = Yc, gc["dX"]
        for _, k in gkeys:
            sums[k] = sums[k] + gc[k].astype(np.float64)
        for k in ("e", "g"):
            got = host(saved[k][sl])
            assert np.all(np.isfinite(got)), f"{k}: non-finite values in rows {t0}.."
            err[k][0] = max(err[k][0], float(np.abs(got - sc[k]).max()))
            err[k][1] = max(err[k][1], float(np.abs(sc[k]).max()))
    tol = TOL["bf16"]
    for k, (e_max, r_max) in err.items():
        print(f"  {k:8s} max|err|/max|ref| = {e_max / r_max:.3e} (tol {tol:g})", flush=True)
        assert e_max <= tol * r_max, k
    assert_close("Y", host(Y), Yr, tol)
    assert_close("dX", host(dX), dXr, tol)
    for k_dev, k_ref in gkeys:
        assert_close(k_dev, host(grads[k_dev]), sums[k_ref], tol)


def test_mlp_B_zero_gives_zero_dA_and_base_output(lm):
    import torch

    cfg = WorkloadConfig(100, "mlp", T=260, H=256, I=384, r=16, alpha=32, dtype="bf16")
    inp = make_mlp_inputs(cfg)
    for k in ("gate", "up", "down"):
        inp[k]["B"] = np.zeros_like(inp[k]["B"])
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d)
    torch.cuda.synchronize()
    for kk in ("dA_gate", "dA_up", "dA_down"):
        assert torch.all(grads[kk] == 0), kk
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"])
    assert_close("Y", host(Y), Yr, TOL["bf16"])


@pytest.mark.parametrize("case", ["A_zero", "s_zero"])
def test_mlp_A_zero_or_scale_zero(lm, case):
    # A = 0: U = 0, so every dB is exactly zero while dA = s X^T (dZ B^T) is not;
    # s = 0: the adapter term, every dA and every dB vanish exactly.  The rest
    # is compared with the oracle.
    import torch

    cfg = WorkloadConfig(101, "mlp", T=300, H=256, I=384, r=16, alpha=32, dtype="bf16")
    inp = make_mlp_inputs(cfg)
    for k in ("gate", "up", "down"):
        if case == "A_zero":
            inp[k]["A"] = np.zeros_like(inp[k]["A"])
        else:
            inp[k]["s"] = 0.0
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d)
    torch.cuda.synchronize()
    zero = ("dB_gate", "dB_up", "dB_down") + (("dA_gate", "dA_up", "dA_down") if case == "s_zero" else ())
    for kk in zero:
        assert torch.all(grads[kk] == 0), kk
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"])
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"])
    assert_close("Y", host(Y), Yr, TOL["bf16"])
    assert_close("dX", host(dX), gr["dX"], TOL["bf16"])
    if case == "A_zero":
        for k_dev, k_ref in (("dA_gate", "dA_g"), ("dA_up", "dA_u"), ("dA_down", "dA_d")):
            assert_close(k_dev, host(grads[k_dev]), gr[k_ref], TOL["bf16"])


def test_mlp_token_permutation(lm):
    # Rows are independent: permuting the tokens permutes the rows of Y, e, g
    # and dX bit for bit; dA and dB change only by their summation order.
    import torch

    cfg = WorkloadConfig(102, "mlp", T=700, H=256, I=640, r=16, alpha=32, dtype="bf16")
    inp = make_mlp_inputs(cfg)
    perm = np.random.default_rng(7).permutation(cfg.T)
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    out = []
    for rows in (np.arange(cfg.T), perm):
        X, dY = dev(inp["X"][rows]), dev(inp["dY"][rows])
        Y, saved = lm.mlp_fwd(X, g, u, d)
        dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d)
        torch.cuda.synchronize()
        out.append((Y, saved, dX, grads))
    (Y0, s0, dX0, g0), (Y1, s1, dX1, g1) = out
    idx = torch.from_numpy(perm).to("cuda:0")
    assert torch.equal(Y0[idx], Y1)
    assert torch.equal(s0["e"][idx], s1["e"])
    assert torch.equal(s0["g"][idx], s1["g"])
    assert torch.equal(dX0[idx], dX1)
    for kk in g0:
        assert_close(kk, host(g1[kk]), host(g0[kk]), TOL["bf16"])


def test_deterministic_repeat(lm):
    import torch

    cfg = WorkloadConfig(101, "mlp", T=300, H=512, I=640, r=16, alpha=32, dtype="bf16")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    outs = []
    for _ in range(2):
        Y, saved = lm.mlp_fwd(X, g, u, d)
        dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d)
        torch.cuda.synchronize()
        outs.append([Y.clone(), dX.clone()] + [grads[k].clone() for k in sorted(grads)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_errors_enqueue_nothing(lm):
    import torch

    X = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda:0")
    A = torch.zeros((256, 16), dtype=torch.bfloat16, device="cuda:0")
    B = torch.zeros((16, 320), dtype=torch.bfloat16, device="cuda:0")
    W = torch.zeros((256, 320), dtype=torch.bfloat16, device="cuda:0")
    p = lm.Proj(A=A, B=B, scale=1.0, W=W)
    with pytest.raises(lm.LoraError) as ei:
        lm.o_fwd(X, p, ws=torch.empty(1, dtype=torch.uint8, device="cuda:0"))
    assert ei.value.status == 5  # LORA_EWORKSPACE
    # dX may be X itself (in place) but not a partly overlapping view of it
    buf = torch.zeros(65 * 256, dtype=torch.bfloat16, device="cuda:0")
    Xv, dXv = buf[:64 * 256].view(64, 256), buf[256:].view(64, 256)
    with pytest.raises(lm.LoraError) as ei:
        lm.o_bwd(torch.zeros((64, 320), dtype=torch.bfloat16, device="cuda:0"), Xv,
                 torch.zeros((64, 16), dtype=torch.bfloat16, device="cuda:0"), p, dX=dXv)
    assert ei.value.status == 6  # LORA_EUNSUPPORTED (dX partly overlaps X)


# ---------------------------------------------------------------------------
# In-place dX: every backward may write dX over X ("LoRA Optimizations",
# "Custom autograd functions"; the unsloth backward hunks write dX into X's
# storage once dA = s X^T P has been formed).  The in-place dX and gradients
# are compared with the oracle, and with the out-of-place call bit for bit
# (same kernels, same order; X is last read by the dA pass, which precedes
# the dX GEMM).
# ---------------------------------------------------------------------------

def _grads_equal(a, b):
    import torch

    assert a.keys() == b.keys()
    for k in a:
        assert torch.equal(a[k], b[k]), k


_MLP_GRADS = (("dA_gate", "dA_g"), ("dB_gate", "dB_g"), ("dA_up", "dA_u"), ("dB_up", "dB_u"),
              ("dA_down", "dA_d"), ("dB_down", "dB_d"))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_inplace_dx_mlp(lm, dt):
    import torch

    cfg = WorkloadConfig(95, "mlp", T=300, H=512, I=640, r=16, alpha=32, dtype=dt, act="swiglu")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"], dt), dev(inp["dY"], dt)
    g, u, d = (proj_dev(inp[k], dt) for k in ("gate", "up", "down"))
    Y, saved = lm.mlp_fwd(X, g, u, d)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d)
    Xi = X.clone()
    dXi, gi = lm.mlp_bwd(dY, Xi, saved, g, u, d, dX=Xi)
    torch.cuda.synchronize()
    assert dXi.data_ptr() == Xi.data_ptr()
    _, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"])
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"])
    tol = TOL[dt]
    assert_close("dX (in place)", host(Xi), gr["dX"], tol)
    for k_dev, k_ref in _MLP_GRADS:
        assert_close(k_dev, host(gi[k_dev]), gr[k_ref], tol)
    assert torch.equal(Xi, dX)
    _grads_equal(grads, gi)


def test_inplace_dx_relu2_mlp(lm):
    import torch

    cfg = WorkloadConfig(96, "relu2", T=300, H=512, I=640, r=16, alpha=32, dtype="bf16")
    inp = make_relu2_inputs(cfg)
    X, dY = dev(inp["X"], "bf16"), dev(inp["dY"], "bf16")
    up, down = (proj_dev(inp[k], "bf16") for k in ("up", "down"))
    Y, saved = lm.relu2_mlp_fwd(X, up, down)
    dX, grads = lm.relu2_mlp_bwd(dY, X, saved, up, down)
    Xi = X.clone()
    _, gi = lm.relu2_mlp_bwd(dY, Xi, saved, up, down, dX=Xi)
    torch.cuda.synchronize()
    _, sr = OL.relu2_mlp_fwd(inp["X"], inp["up"], inp["down"])
    gr = OL.relu2_mlp_bwd(inp["dY"], inp["X"], sr, inp["up"], inp["down"])
    tol = TOL["bf16"]
    assert_close("dX (in place)", host(Xi), gr["dX"], tol)
    for k_dev, k_ref in (("dA_up", "dA_u"), ("dB_up", "dB_u"), ("dA_down", "dA_d"), ("dB_down", "dB_d")):
        assert_close(k_dev, host(gi[k_dev]), gr[k_ref], tol)
    assert torch.equal(Xi, dX)
    _grads_equal(grads, gi)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_inplace_dx_qkv_o(lm, dt):
    import torch

    cfg = WorkloadConfig(97, "attn", T=300, H=512, r=16, alpha=32, dtype=dt, Nq=512, Nk=192, Nv=128)
    inp = make_attn_inputs(cfg)
    X = dev(inp["X"], dt)
    q, k, v = (proj_dev(inp[n], dt) for n in ("q", "k", "v"))
    Q, K, V, U = lm.qkv_fwd(X, q, k, v)
    dQ, dK, dV = (dev(inp[n], dt) for n in ("dQ", "dK", "dV"))
    dX, grads = lm.qkv_bwd(dQ, dK, dV, X, U, q, k, v)
    Xi = X.clone()
    _, gi = lm.qkv_bwd(dQ, dK, dV, Xi, U, q, k, v, dX=Xi)
    Xo = dev(inp["Xo"], dt)
    o = proj_dev(inp["o"], dt)
    Yo, Uo = lm.o_fwd(Xo, o)
    dO = dev(inp["dO"], dt)
    dXo, dAo, dBo = lm.o_bwd(dO, Xo, Uo, o)
    Xoi = Xo.clone()
    _, dAoi, dBoi = lm.o_bwd(dO, Xoi, Uo, o, dX=Xoi)
    torch.cuda.synchronize()
    _, sr = OL.qkv_fwd(inp["X"], inp["q"], inp["k"], inp["v"])
    gr = OL.qkv_bwd(inp["dQ"], inp["dK"], inp["dV"], inp["X"], sr, inp["q"], inp["k"], inp["v"])
    _, so = OL.o_fwd(inp["Xo"], inp["o"])
    go = OL.o_bwd(inp["dO"], inp["Xo"], so, inp["o"])
    tol = TOL[dt]
    assert_close("dX (in place)", host(Xi), gr["dX"], tol)
    for n in ("dA_q", "dB_q", "dA_k", "dB_k", "dA_v", "dB_v"):
        assert_close(n, host(gi[n]), gr[n], tol)
    assert_close("dX_o (in place)", host(Xoi), go["dX"], tol)
    assert_close("dA_o", host(dAoi), go["dA"], tol)
    assert_close("dB_o", host(dBoi), go["dB"], tol)
    assert torch.equal(Xi, dX)
    _grads_equal(grads, gi)
    assert torch.equal(Xoi, dXo)
    assert torch.equal(dAoi, dAo) and torch.equal(dBoi, dBo)


def test_non_default_stream(lm):
    """A call on a caller's stream: outputs and workspace are allocated on that
    stream, so memory the current stream allocates and overwrites right after
    the call (while the call's kernels may still run) cannot be a buffer the
    call uses.  Results are checked against the oracle after the stream ends."""
    import torch

    cfg = WorkloadConfig(107, "mlp", T=300, H=512, I=1088, r=16, alpha=32, dtype="bf16", act="swiglu")
    inp = make_mlp_inputs(cfg)
    X, dY = dev(inp["X"]), dev(inp["dY"])
    g, u, d = (proj_dev(inp[k]) for k in ("gate", "up", "down"))
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    Y, saved = lm.mlp_fwd(X, g, u, d, stream=s)
    dX, grads = lm.mlp_bwd(dY, X, saved, g, u, d, stream=s)
    junk = [torch.full((1 << 22,), float("nan"), dtype=torch.float32, device="cuda:0") for _ in range(16)]
    s.synchronize()
    torch.cuda.synchronize()
    del junk
    Yr, sr = OL.mlp_fwd(inp["X"], inp["gate"], inp["up"], inp["down"])
    gr = OL.mlp_bwd(inp["dY"], inp["X"], sr, inp["gate"], inp["up"], inp["down"])
    tol = TOL["bf16"]
    assert_close("Y", host(Y), Yr, tol)
    assert_close("dX", host(dX), gr["dX"], tol)
    for k_dev, k_ref in _MLP_GRADS:
        assert_close(k_dev, host(grads[k_dev]), gr[k_ref], tol)
