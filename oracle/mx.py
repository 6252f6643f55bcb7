"""MX (microscaling) FP8 quantization and the block-scaled matrix product, plainly
(test infrastructure only, like the rest of this package).

The pages name the step in one phrase: after fp32, take the trainer's precision down
to fp16 and below ("1000 行 C 代码完成 GPT-2 训练的 LLM.c", the paragraph on what comes
after the CUDA port).  Below 16 bits the format read here is OCP MXFP8 with E4M3
elements, the block-scaled 8-bit format gfx950's matrix cores take natively:

* an E4M3 element has a sign bit, 4 exponent bits (bias 7) and 3 mantissa bits;
  exponent field 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no
  infinity, so the largest magnitude is 1.75 * 2^8 = 448;
* a block is 32 consecutive values along the reduction dimension k, sharing one
  scale 2^e stored as an 8-bit biased exponent (E8M0: e + 127, e in [-127, 127]);
* the scale of a block with largest magnitude amax is the smallest power of two 2^e
  with amax / 2^e <= 448, so the largest element lands in (224, 448] and nothing is
  clipped (the OCP specification's own example rule, 2^(floor(log2 amax) - 8), would
  clip block maxima with a mantissa of 1.75 or more by up to an eighth); elements are
  x / 2^e rounded to the nearest E4M3 value (ties to the even mantissa, magnitudes
  above 448 clamped to 448, which this scale never needs); an all-zero block, or one
  below E8M0's range, gets e = -127.

The product of two MX operands is the sum over k of the dequantized elements
(element value times its block's scale).  Everything is float64 numpy.
Pinned in tests/test_mx_oracle.py (format table, rounding, clamping, scale range,
lossless blocks, products of exactly representable operands).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
EMAX_E4M3 = 8
MAX_E4M3 = 448.0


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code from the format's fields."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3 = np.array([e4m3_value(c) for c in range(256)])
# the 127 finite non-negative codes 0x00 .. 0x7E in increasing order of value
_POS_CODES = np.arange(0x7F)
_POS_VALS = E4M3[_POS_CODES]


def e4m3_encode(v):
    """Nearest E4M3 code to each value (ties: the code with the even mantissa; above
    448 in magnitude: 448; the sign bit is the input's, so small negatives give -0)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), MAX_E4M3)
    hi = np.clip(np.searchsorted(_POS_VALS, a, side="left"), 0, _POS_VALS.size - 1)
    lo = np.clip(hi - 1, 0, None)
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    # the sign is kept, also when the magnitude rounds to zero (-0 is code 0x80)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def block_exponent(amax):
    """The shared exponent e of blocks with largest magnitude amax: the smallest
    integer with amax <= 448 * 2^e."""
    amax = np.asarray(amax, dtype=np.float64)
    _, p = np.frexp(amax)  # amax = f 2^p, f in [0.5, 1)  =>  floor(log2 amax) = p - 1
    e = p - 1 - EMAX_E4M3  # amax / 2^e in [256, 512), exactly (a power-of-two scaling)
    e = e + (np.ldexp(amax, -e) > MAX_E4M3)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize(x):
    """MX quantization of x [rows, K] along its last axis (K a multiple of 32).
    Returns (codes uint8 [rows, K], e int64 [rows, K / 32])."""
    x = np.asarray(x, dtype=np.float64)
    R, K = x.shape
    assert K % BLOCK == 0
    xb = x.reshape(R, K // BLOCK, BLOCK)
    e = block_exponent(np.abs(xb).max(axis=2))
    codes = e4m3_encode(xb * np.ldexp(1.0, -e)[:, :, None])
    return codes.reshape(R, K), e


def dequantize(codes, e):
    R, K = codes.shape
    v = E4M3[codes.astype(np.int64)].reshape(R, K // BLOCK, BLOCK)
    return (v * np.ldexp(1.0, e)[:, :, None]).reshape(R, K)


def matmul(qa, ea, qb, eb):
    """A B^T for MX operands A [M, K] and B [N, K] (dequantized, float64)."""
    return dequantize(qa, ea) @ dequantize(qb, eb).T
