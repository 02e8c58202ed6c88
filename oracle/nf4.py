"""Oracle for the NF4 storage format of frozen base weights: quantize,
unpack and dequantize (float32 and bfloat16).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("loralei" README, section "Use", QLoRA paragraphs): the
frozen weights of the selected linear layers are stored as NF4 codes in blocks
of 64 elements whose scales are themselves quantized ("double-scale
reconstruction") in scaler blocks of 256 blocks; a weight's element count must
be divisible by 64 * 256; the fused kernels unpack the codes and rebuild the
two-level scale inside the matmul.  The Axolotl optimizations guide names
bitsandbytes 4-bit loading for QLoRA.

What the pages leave open is fixed here (plainest reading, listed in the design
notes):

1. Blocks are 64 consecutive elements of the row-major flattened weight
   ``W [in, out]``; scaler blocks are 256 consecutive blocks.
2. ``a_b = max |w|`` over the block (exact).
3. Code ``q_j = argmin_i |fl32(w_j / a_b) - c_i|`` over the 16 NF4 levels
   ``c_i`` (float32 arithmetic, ties to the lower index); an all-zero block
   uses x = 0, i.e. code 7 (the exact zero level).
4. ``mu`` = float32 of (S / nblocks), where S is the float64 sum of all
   ``a_b`` taken as: the 256 absmaxes of each scaler block summed in
   ascending order, then the scaler-block sums added in ascending order.
5. Per scaler block: ``d_b = fl32(a_b - mu)``, ``m = max |d_b|``,
   ``s2 = fl32(m / 127)``, ``q8_b = clamp(rint(fl32(d_b / s2)), -127, 127)``
   (int8, round half to even), or 0 when s2 == 0.
6. Packing: byte ``j`` holds code ``2j`` in bits 7..4 and ``2j+1`` in bits 3..0.
7. Dequant: ``a'_b = fl32(fl32(q8_b * s2) + mu)``, ``w'_j = fl32(c_{q_j} * a'_b)``;
   the bfloat16 form is ``w'_j`` rounded to nearest-even.

Codebook: the 16 NF4 levels of the QLoRA paper (Dettmers et al., 2023,
appendix), asymmetric standard-normal quantiles normalised to [-1, 1] with an
exact zero; a pin regenerates them from the paper's construction.

Parity pins (tests/test_oracle_nf4.py): codebook construction and shape,
exact round trip of representable blocks, brute-force code choice against an
independent sorted-midpoint search, reconstruction error bounds, a hand-built
block, divisibility rules.  Byte compatibility with TorchAO or bitsandbytes is
parity unpinned (neither library is available).
"""
from __future__ import annotations

import numpy as np

BLOCK = 64
SCALER_BLOCK = 256

NF4_LEVELS = np.array(
    [
        -1.0, -0.6961928, -0.5250731, -0.3949175,
        -0.2844414, -0.1847734, -0.0910500, 0.0,
        0.0795803, 0.1609302, 0.2461123, 0.3379152,
        0.4407098, 0.5626170, 0.7229568, 1.0,
    ],
    dtype=np.float32,
)


def check_shape(numel: int) -> None:
    if numel % (BLOCK * SCALER_BLOCK) != 0:
        raise ValueError(f"NF4 needs numel divisible by {BLOCK * SCALER_BLOCK}, got {numel}")


def block_absmax(w_flat: np.ndarray) -> np.ndarray:
    """Step 2: exact max |w| of each block of 64 consecutive elements."""
    return np.abs(w_flat.reshape(-1, BLOCK)).max(axis=1).astype(np.float32)


def nearest_codes(x: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """Step 3: index of the nearest NF4 level to each float32 ``x`` (first
    minimum wins, i.e. ties go to the lower index).  Brute force over all 16
    levels."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(x.shape[0], dtype=np.uint8)
    for i in range(0, x.shape[0], chunk):
        xs = x[i:i + chunk]
        dist = np.abs(xs[:, None] - NF4_LEVELS[None, :])  # float32
        out[i:i + chunk] = np.argmin(dist, axis=1).astype(np.uint8)
    return out


def global_mean_absmax(absmax: np.ndarray) -> np.float32:
    """Step 4: mu = fl32(S / nblocks), S summed in float64 per scaler block in
    ascending order, then over scaler blocks in ascending order."""
    a = absmax.astype(np.float64).reshape(-1, SCALER_BLOCK)
    per_sb = np.cumsum(a, axis=1)[:, -1]
    total = np.cumsum(per_sb)[-1]
    return np.float32(total / np.float64(absmax.shape[0]))


def double_quantize(absmax: np.ndarray, mu: np.float32):
    """Step 5: int8 codes of the mean-centred absmaxes with one float32 scale
    per scaler block.  Returns (q8 int8 [nblocks], s2 float32 [nscaler])."""
    d = (absmax - mu).astype(np.float32).reshape(-1, SCALER_BLOCK)
    m = np.abs(d).max(axis=1)
    s2 = (m / np.float32(127)).astype(np.float32)
    q8 = np.zeros_like(d, dtype=np.int8)
    nz = s2 > 0
    ratio = (d[nz] / s2[nz][:, None]).astype(np.float32)
    q8[nz] = np.clip(np.rint(ratio), -127, 127).astype(np.int8)
    return q8.reshape(-1), s2


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Step 6: two codes per byte, even element in the high nibble."""
    c = codes.astype(np.uint8).reshape(-1, 2)
    return ((c[:, 0] << 4) | c[:, 1]).astype(np.uint8)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of step 6: uint8 codes in element order."""
    p = packed.astype(np.uint8).reshape(-1)
    out = np.empty(p.shape[0] * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


def quantize(w: np.ndarray) -> dict:
    """Quantize a float32 weight (any shape; flattened row-major) to NF4.

    Returns dict(codes=uint8 [numel/2], q8=int8 [numel/64],
    s2=float32 [numel/16384], mu=float32 scalar, shape=w.shape)."""
    w_flat = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    check_shape(w_flat.shape[0])
    a = block_absmax(w_flat)
    a_rep = np.repeat(a, BLOCK)
    safe = np.where(a_rep > 0, a_rep, np.float32(1))
    x = np.where(a_rep > 0, (w_flat / safe).astype(np.float32), np.float32(0))
    codes = nearest_codes(x)
    mu = global_mean_absmax(a)
    q8, s2 = double_quantize(a, mu)
    return dict(codes=pack_codes(codes), q8=q8, s2=s2, mu=np.float32(mu), shape=tuple(w.shape))


def reconstruct_absmax(q8: np.ndarray, s2: np.ndarray, mu) -> np.ndarray:
    """Step 7, first half: a'_b = fl32(fl32(q8_b * s2) + mu)."""
    s2_rep = np.repeat(np.asarray(s2, np.float32), SCALER_BLOCK)
    prod = (q8.astype(np.float32) * s2_rep).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


def dequantize(q: dict, out: str = "f32") -> np.ndarray:
    """Step 7: w'_j = fl32(c[q_j] * a'_b); ``out="bf16"`` rounds w' to the
    nearest bfloat16 (ties to even) and returns it widened to float32."""
    codes = unpack_codes(q["codes"])
    a_prime = reconstruct_absmax(q["q8"], q["s2"], q["mu"])
    w = (NF4_LEVELS[codes] * np.repeat(a_prime, BLOCK)).astype(np.float32)
    if out == "bf16":
        w = round_to_bf16(w)
    elif out != "f32":
        raise ValueError(out)
    return w.reshape(q["shape"])


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32).reshape(np.shape(x))
