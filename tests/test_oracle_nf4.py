"""Pins of the NF4 oracle.

* The codebook: the QLoRA paper's construction (asymmetric standard-normal
  quantiles with an exact zero) regenerated with scipy, the printed values
  (golden file), and the shape facts (16 increasing levels, -1, 0, 1).
* A block built by hand whose codes were worked out on paper (golden file),
  including an exact tie.
* Exact round trip of blocks made of representable values (every level times
  a shared power of two): codes, scales and float32 dequant reproduce the
  input bit for bit.
* The code choice against an independent search (sorted midpoints), on random
  values; reconstruction-error bounds; divisibility and packing rules.
"""
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import nf4 as Q


def _read_golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_codebook_shape_facts():
    c = Q.NF4_LEVELS
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1 and c[7] == 0 and c[15] == 1
    assert np.sum(c < 0) == 7 and np.sum(c > 0) == 8


def test_codebook_matches_qlora_construction(golden_dir):
    """QLoRA (Dettmers et al. 2023): 8 positive quantiles of N(0,1) over
    [delta, 1/2) and 7 negative ones, plus one exact zero, normalised to
    [-1, 1]; delta = 1 - (1/32 + 1/30)/2 puts the extreme quantiles at the
    midpoints of the outer probability bins."""
    delta = 1 - 0.5 * (1 / 32 + 1 / 30)
    pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    levels = np.sort(np.concatenate([pos, [0.0], neg]))
    levels /= levels.max()
    # the paper prints 7 decimals; the construction agrees to that precision
    assert np.abs(levels - Q.NF4_LEVELS.astype(np.float64)).max() < 2e-7
    printed = np.array([float(r[0]) for r in _read_golden(golden_dir, "nf4_levels_qlora_paper.txt")],
                       dtype=np.float32)
    assert np.array_equal(printed, Q.NF4_LEVELS)


def test_hand_built_block(golden_dir):
    rows = _read_golden(golden_dir, "nf4_hand_block.txt")
    vals = np.array([float(r[0]) for r in rows], dtype=np.float32)
    want = np.array([int(r[1]) for r in rows], dtype=np.uint8)
    assert vals.shape == (64,)
    w = np.tile(vals, Q.SCALER_BLOCK)  # 16384 elements: one scaler block
    q = Q.quantize(w)
    codes = Q.unpack_codes(q["codes"])
    assert np.array_equal(codes[:64], want)
    assert q["mu"] == np.float32(2.0)
    assert np.all(q["q8"] == 0) and np.all(q["s2"] == 0)
    # byte 0 packs element 0 (code 15) high and element 1 (code 0) low
    assert q["codes"][0] == 0xF0


def _representable_blocks(rng, nblocks, k):
    """Blocks whose every value is c_i * 2^k, each block holding +2^k."""
    codes = rng.integers(0, 16, size=(nblocks, Q.BLOCK)).astype(np.uint8)
    codes[:, rng.integers(0, Q.BLOCK)] = 15
    w = Q.NF4_LEVELS[codes] * np.float32(2.0 ** k)
    return w.astype(np.float32), codes


@pytest.mark.parametrize("k", [-7, 0, 3])
def test_exact_round_trip_of_representable_blocks(k):
    rng = np.random.default_rng(10 + k)
    w, codes = _representable_blocks(rng, 2 * Q.SCALER_BLOCK, k)
    q = Q.quantize(w.reshape(128, -1))
    assert np.array_equal(Q.unpack_codes(q["codes"]), codes.reshape(-1))
    assert q["mu"] == np.float32(2.0 ** k)
    assert np.all(q["q8"] == 0) and np.all(q["s2"] == 0)
    deq = Q.dequantize(q, "f32").reshape(-1)
    assert np.array_equal(deq.view(np.uint32), w.reshape(-1).view(np.uint32))
    # bf16 of representable-in-bf16 values is the identity too (levels * 2^k
    # carry up to 24 significant bits, so compare against explicit RNE)
    deq16 = Q.dequantize(q, "bf16").reshape(-1)
    assert np.all(np.abs(deq16 - w.reshape(-1)) <= np.abs(w.reshape(-1)) * 2.0 ** -8)


def _codes_by_midpoints(x):
    """Independent code search: binary search among the 15 midpoints."""
    c = Q.NF4_LEVELS.astype(np.float64)
    mids = (c[:-1] + c[1:]) / 2
    return np.searchsorted(mids, x.astype(np.float64), side="left").astype(np.uint8)


def test_code_choice_against_sorted_midpoints():
    rng = np.random.default_rng(11)
    x = np.clip(rng.standard_normal(200_000).astype(np.float32) * 0.5, -1, 1)
    a = Q.nearest_codes(x)
    b = _codes_by_midpoints(x)
    diff = np.nonzero(a != b)[0]
    # disagreement is only possible within float32 rounding of a midpoint
    c = Q.NF4_LEVELS.astype(np.float64)
    for i in diff:
        lo, hi = sorted((a[i], b[i]))
        assert hi == lo + 1
        assert abs(x[i] - (c[lo] + c[hi]) / 2) < 1e-6
    assert diff.size < 5
    # exhaustive: each chosen level is a nearest one
    dist = np.abs(x[:, None].astype(np.float64) - c[None, :])
    assert np.all(dist[np.arange(x.size), a] <= dist.min(axis=1) + 1e-7)


def test_quantize_random_weight_error_bounds():
    rng = np.random.default_rng(12)
    n_in, n_out = 256, 128  # 32768 elements = 2 scaler blocks
    w = (rng.standard_normal((n_in, n_out)) / np.sqrt(n_in)).astype(np.float32)
    q = Q.quantize(w)
    assert q["codes"].shape == (w.size // 2,) and q["codes"].dtype == np.uint8
    assert q["q8"].shape == (w.size // 64,) and q["q8"].dtype == np.int8
    assert q["s2"].shape == (w.size // 16384,) and q["s2"].dtype == np.float32
    assert np.all(np.abs(q["q8"].astype(int)) <= 127)
    # each scaler block uses the full int8 range at its extreme block
    assert np.all(np.abs(q["q8"].reshape(-1, 256)).max(axis=1) == 127)
    a = Q.block_absmax(w.reshape(-1))
    mu64 = a.astype(np.float64).mean()
    assert abs(q["mu"] - mu64) <= 2 * np.spacing(np.float32(mu64))
    a_rec = Q.reconstruct_absmax(q["q8"], q["s2"], q["mu"])
    s2_rep = np.repeat(q["s2"], 256).astype(np.float64)
    assert np.all(np.abs(a_rec - a) <= 0.5 * s2_rep * (1 + 1e-5) + 4 * np.spacing(a))
    deq = Q.dequantize(q, "f32").reshape(-1)
    c = Q.NF4_LEVELS.astype(np.float64)
    gap = np.diff(c).max()
    bound = 0.5 * gap * np.repeat(np.maximum(a, a_rec), 64) + np.repeat(np.abs(a - a_rec), 64) + 1e-7
    assert np.all(np.abs(deq - w.reshape(-1)) <= bound)
    deq16 = Q.dequantize(q, "bf16").reshape(-1)
    assert np.all(np.abs(deq16 - deq) <= np.abs(deq) * 2.0 ** -8)  # half a bf16 ulp


def test_zero_block_gets_code_seven_and_divisibility_rule():
    w = np.zeros(16384, np.float32)
    w[64:128] = np.linspace(-1, 1, 64, dtype=np.float32)
    q = Q.quantize(w)
    codes = Q.unpack_codes(q["codes"])
    assert np.all(codes[:64] == 7) and np.all(codes[128:] == 7)
    with pytest.raises(ValueError):
        Q.quantize(np.zeros(16384 + 64, np.float32))


def test_pack_unpack_round_trip_and_nibble_order():
    codes = np.arange(16, dtype=np.uint8).repeat(2)
    packed = Q.pack_codes(codes)
    assert packed[0] == 0x00 and packed[1] == 0x11 and packed[15] == 0xFF
    odd = np.array([3, 12], dtype=np.uint8)
    assert Q.pack_codes(odd)[0] == 0x3C
    rng = np.random.default_rng(13)
    c = rng.integers(0, 16, 4096).astype(np.uint8)
    assert np.array_equal(Q.unpack_codes(Q.pack_codes(c)), c)


def test_bf16_rounding_is_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)  # bf16 spacing at 1
    x = np.array([one + ulp / 2, one + ulp * 1.5, one + ulp / 2 + 2.0 ** -20, -(one + ulp / 2)],
                 dtype=np.float32)
    r = Q.round_to_bf16(x)
    assert r[0] == one                # tie -> even (1.0)
    assert r[1] == one + 2 * ulp      # tie -> even (1 + 2 ulp)
    assert r[2] == one + ulp          # above the tie -> up
    assert r[3] == -one
