"""Pins of the MX FP8 oracle (oracle/mx.py) to the E4M3 / E8M0 format definitions
and to closed forms of the block-scaled product."""
import numpy as np

from oracle import mx


def test_e4m3_table_landmarks():
    E = mx.E4M3
    assert E[0x00] == 0.0 and E[0x80] == 0.0 and np.signbit(E[0x80])
    assert np.isnan(E[0x7F]) and np.isnan(E[0xFF]) and np.isnan(E).sum() == 2
    assert E[0x7E] == 448.0 and E[0xFE] == -448.0          # 1.75 * 2^8
    assert E[0x38] == 1.0 and E[0x40] == 2.0 and E[0x30] == 0.5
    assert E[0x08] == 2.0 ** -6                          # smallest normal
    assert E[0x01] == 2.0 ** -9 and E[0x07] == 7 * 2.0 ** -9   # subnormals
    finite = E[~np.isnan(E)]
    assert np.unique(finite).size == 253                 # 254 finite codes, +0 == -0
    assert np.all(np.diff(E[:0x7F]) > 0)                  # codes 0..126 increase
    np.testing.assert_array_equal(E[0x80:0xFF], -E[0x00:0x7F])


def test_encode_round_trip_ties_and_clamp():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(mx.e4m3_encode(mx.E4M3[codes]), codes)   # -0 included
    assert mx.e4m3_encode(-2.0 ** -12) == 0x80 and mx.e4m3_encode(2.0 ** -12) == 0x00
    # midpoints go to the even mantissa: 1 + 1/16 -> 1 (m = 0); 1 + 3/16 -> 1.25 (m = 2)
    assert mx.e4m3_encode(1.0625) == 0x38 and mx.e4m3_encode(1.1875) == 0x3A
    assert mx.e4m3_encode(-1.1875) == 0xBA
    # just off a midpoint goes to the nearer value
    assert mx.e4m3_encode(1.0625 + 1e-9) == 0x39 and mx.e4m3_encode(1.0625 - 1e-9) == 0x38
    # between 416 and 448 the midpoint 432 ties to 448 (m = 6 is even), above 448 clamps
    assert mx.e4m3_encode(432.0) == 0x7E and mx.e4m3_encode(431.9) == 0x7D
    assert mx.e4m3_encode(1e6) == 0x7E and mx.e4m3_encode(-500.0) == 0xFE
    # below half the smallest subnormal: zero (the tie 2^-10 goes to the even code 0)
    assert mx.e4m3_encode(2.0 ** -10) == 0x00 and mx.e4m3_encode(2.0 ** -10 * 1.001) == 0x01
    # brute force: the chosen value is a nearest finite value to the clamped input
    rng = np.random.default_rng(0)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-12, 10, 20000))
    got = mx.E4M3[mx.e4m3_encode(v)]
    fin = np.unique(mx.E4M3[~np.isnan(mx.E4M3)])
    c = np.clip(v, -448, 448)
    best = np.abs(fin[None, :] - c[:, None]).min(axis=1)
    np.testing.assert_array_equal(np.abs(got - c), best)


def test_block_exponent_is_the_smallest_scale_that_does_not_clip():
    rng = np.random.default_rng(1)
    amax = np.abs(rng.standard_normal(5000)) * np.exp2(rng.integers(-40, 40, 5000))
    e = mx.block_exponent(amax)
    r = amax * np.exp2(-e.astype(float))
    assert np.all((r > 224) & (r <= 448))                      # one scale smaller would exceed 448
    assert mx.block_exponent(np.array([448.0]))[0] == 0        # 448 = 1.75 * 2^8 fits exactly
    assert mx.block_exponent(np.array([448.0 * (1 + 2.0 ** -20)]))[0] == 1
    assert mx.block_exponent(np.array([256.0]))[0] == 0 and mx.block_exponent(np.array([224.0]))[0] == -1
    assert mx.block_exponent(np.array([1.0]))[0] == -8
    assert mx.block_exponent(np.array([0.0]))[0] == -127
    assert mx.block_exponent(np.array([2.0 ** -140]))[0] == -127   # clamped to E8M0's range


def test_quantize_error_bounds_and_lossless_blocks():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 128)) * np.exp2(rng.integers(-6, 6, (16, 1)))
    q, e = mx.quantize(x)
    d = mx.dequantize(q, e)
    scale = np.repeat(np.exp2(e.astype(float)), 32, axis=1)
    # each element is within half a step of the E4M3 grid at its magnitude (3 bits)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(x) / scale, 2.0 ** -6))) - 3) * scale
    assert np.all(np.abs(d - x) <= step / 2 + 1e-300)
    # a block of E4M3 values times 2^s whose largest magnitude is 448 is kept exactly
    codes = rng.integers(0, 0x7F, (4, 64)).astype(np.uint8) | (rng.integers(0, 2, (4, 64)) << 7).astype(np.uint8)
    codes[:, 0], codes[:, 32] = 0x7E, 0x7E
    vals = mx.E4M3[codes] * np.exp2(np.array([[-3.0], [0.0], [5.0], [-20.0]]))
    q2, e2 = mx.quantize(vals)
    np.testing.assert_array_equal(mx.dequantize(q2, e2), vals)
    # all-zero block
    qz, ez = mx.quantize(np.zeros((1, 32)))
    assert not qz.any() and ez[0, 0] == -127


def test_block_scaled_product_of_representable_operands_is_exact():
    rng = np.random.default_rng(3)
    def representable(R, K):
        c = rng.integers(0, 0x7F, (R, K)) | (rng.integers(0, 2, (R, K)) << 7)
        c[:, ::32] = 0x7E   # each block's maximum is 448, so quantization keeps every value
        return mx.E4M3[c] * np.exp2(rng.integers(-4, 4, (R, 1)).astype(float))
    a, b = representable(24, 96), representable(40, 96)
    qa, ea = mx.quantize(a)
    qb, eb = mx.quantize(b)
    np.testing.assert_array_equal(mx.matmul(qa, ea, qb, eb), a @ b.T)
    # a mistake in the block exponent (one block off by one) would show
    eb2 = eb.copy()
    eb2[0, 1] += 1
    assert not np.array_equal(mx.matmul(qa, ea, qb, eb2), a @ b.T)
