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


# ---------------------------------------------------------------------------- MX mode of the
# C++ oracle: its encode / decode round trip and the operands of each forward product

def _bf16(x):
    """Round-to-nearest-even bf16 of float32-representable values (torch's conversion)."""
    import torch
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _mx_operand(x):
    """The operand an MX product multiplies, from oracle/mx.py's table-based encoder:
    bf16 values, zero-padded to whole 32-blocks, encoded and decoded."""
    x = _bf16(x)
    R, K = x.shape
    Kp = (K + 31) // 32 * 32
    xp = np.pad(x, ((0, 0), (0, Kp - K)))
    return mx.dequantize(*mx.quantize(xp))[:, :K]


def test_cpp_mx_roundtrip_matches_the_table_encoder():
    import oracle
    rng = np.random.default_rng(11)
    for rows, K in [(7, 96), (5, 200), (3, 33), (1, 8)]:
        x = (rng.standard_normal((rows, K)) * np.exp2(rng.integers(-20, 20, (rows, K)))).astype(np.float32)
        x[0, :4] = [0.0, -0.0, 1e-40, -3e-39]        # zeros and fp32 subnormals
        if K >= 64:
            x[1, 32:64] = 0.0                          # an all-zero block
            x[2, 32:40] = [1.0625, 1.1875, 432.0, 448.0, -0.5, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10]
        got = oracle.mx_roundtrip(x.astype(np.float64))
        ref = _mx_operand(x)
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def test_mx_mode_multiplies_the_encoded_operands_of_each_forward_product():
    # In MX mode each of the five forward products (qkv, attention projection, c_fc,
    # c_fc projection, tied lm_head) multiplies its bf16 input and weight through the MX
    # encoding; everything between the products is the plain forward pass.
    import oracle
    import synth
    m = synth.ModelShape(16, 97, 2, 2, 64)
    w = synth.Workload("mx_oracle", m, 2, 16, "bf16", "uniform", index=60)
    p = synth.init_params(m).astype(np.float64)
    rng = np.random.default_rng(60)
    offs = synth.param_offsets(m)
    for name, (o, n) in offs.items():
        if name.endswith(".b"):
            p[o:o + n] = 0.1 * rng.standard_normal(n)
    x, y = synth.inputs_targets(w)
    o = oracle.Oracle(m, w.B, w.T, "f64")
    o.set("params", p)
    loss_plain = o.forward(x, y)
    o.set_mx(True)
    loss_mx = o.forward(x, y)
    C, BT = m.channels, w.B * w.T

    def W(name):
        off, n = offs[name]
        return p[off:off + n]

    def check(out, inp, wname, bname, rows, IC, OC):
        Wm = W(wname).reshape(OC, IC)
        ref = _mx_operand(inp.reshape(rows, IC)) @ _mx_operand(Wm).T
        if bname:
            ref = ref + W(bname)
        np.testing.assert_allclose(out.reshape(rows, OC), ref, rtol=1e-12, atol=1e-12)

    for l in range(m.num_layers):
        h = f"h{l}."
        check(o.act("qkv", l), o.act("ln1", l), h + "qkv.w", h + "qkv.b", BT, C, 3 * C)
        resid_in = o.act("encoded") if l == 0 else o.act("residual3", l - 1)
        proj = o.act("residual2", l) - resid_in
        check(proj, o.act("atty", l), h + "proj.w", h + "proj.b", BT, C, C)
        check(o.act("fch", l), o.act("ln2", l), h + "fc.w", h + "fc.b", BT, C, 4 * C)
        fcp = o.act("residual3", l) - o.act("residual2", l)
        check(fcp, o.act("fch_gelu", l), h + "fcproj.w", h + "fcproj.b", BT, 4 * C, C)
    check(o.act("logits"), o.act("lnf"), "wte", None, BT, C, m.vocab_size)
    # the encoding is really applied (3 mantissa bits: the loss moves)
    assert loss_mx != loss_plain
    o.close()


def test_cpp_mx_input_gradient_product_matches_the_table_encoder():
    # dinp = dout w with dout's rows and w's columns (the rows of w^T) encoded in
    # blocks of 32 along the contraction; OC = 40 leaves a partial block, IC = 24 is
    # not a multiple of anything in particular.
    import oracle
    rng = np.random.default_rng(12)
    for N, IC, OC in [(6, 24, 40), (3, 64, 96), (2, 8, 33)]:
        dout = (rng.standard_normal((N, OC)) * np.exp2(rng.integers(-8, 8, (N, OC)))).astype(np.float32)
        # rows of w at very different scales: a block along OC then spans magnitudes
        # 2^20 apart (its small values land on E4M3's subnormal steps), a block along
        # IC does not, so the two directions encode differently
        w = (rng.standard_normal((OC, IC)) * 0.02 * np.exp2(rng.integers(-10, 10, (OC, 1)))).astype(np.float32)
        ref = _mx_operand(dout) @ _mx_operand(w.T).T
        got = oracle.matmul_backward_input_mx(dout, w)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
        # a transposed reading (blocks along IC instead of OC) is a different product
        wrong = _mx_operand(dout) @ _mx_operand(w)
        assert not np.allclose(got, wrong, rtol=1e-9, atol=1e-12)


def test_mx_mode_2_encodes_the_operands_of_each_input_gradient_product():
    # MX mode 2: the backward pass's input-gradient products of the five forward
    # products multiply MX-encoded operands (the upstream gradient's rows and the
    # weight's columns, blocks of 32 along the layer's outputs); the weight gradients
    # and everything else keep the plain values (straight-through).
    import oracle
    import synth
    m = synth.ModelShape(16, 97, 2, 2, 64)
    w = synth.Workload("mx_dx_oracle", m, 2, 16, "bf16", "uniform", index=61)
    p = synth.init_params(m).astype(np.float64)
    rng = np.random.default_rng(61)
    offs = synth.param_offsets(m)
    for name, (off, n) in offs.items():
        if name.endswith(".b"):
            p[off:off + n] = 0.1 * rng.standard_normal(n)
    x, y = synth.inputs_targets(w)
    o = oracle.Oracle(m, w.B, w.T, "f64")
    o.set("params", p)
    o.set_mx(1)
    loss1 = o.forward(x, y)
    o.backward()
    g1 = o.get("grads")
    o.set_mx(2)
    loss2 = o.forward(x, y)
    o.backward()
    g2 = o.get("grads")
    assert loss1 == loss2          # the forward pass is the same in modes 1 and 2
    assert not np.array_equal(g1, g2)
    C, BT, V = m.channels, w.B * w.T, m.vocab_size

    def W(name):
        off, n = offs[name]
        return p[off:off + n]

    def check_dx(dinp, dout, wname, IC, OC):
        Wm = W(wname).reshape(OC, IC)
        ref = _mx_operand(dout.reshape(BT, OC)) @ _mx_operand(Wm.T).T
        np.testing.assert_allclose(dinp.reshape(BT, IC), ref, rtol=1e-12, atol=1e-13)

    def check_dw(gname, dout, inp, IC, OC):
        off, n = offs[gname]
        ref = dout.reshape(BT, OC).T @ inp.reshape(BT, IC)
        np.testing.assert_allclose(g2[off:off + n].reshape(OC, IC), ref, rtol=1e-10, atol=1e-13)

    for l in range(m.num_layers):
        h = f"h{l}."
        check_dx(o.act("dln1", l), o.act("dqkv", l), h + "qkv.w", C, 3 * C)
        check_dx(o.act("datty", l), o.act("dattproj", l), h + "proj.w", C, C)
        check_dx(o.act("dfch_gelu", l), o.act("dfcproj", l), h + "fcproj.w", 4 * C, C)
        check_dx(o.act("dln2", l), o.act("dfch", l), h + "fc.w", C, 4 * C)
        check_dw(h + "qkv.w", o.act("dqkv", l), o.act("ln1", l), C, 3 * C)
        check_dw(h + "fcproj.w", o.act("dfcproj", l), o.act("fch_gelu", l), 4 * C, C)
    check_dx(o.act("dlnf"), o.act("dlogits"), "wte", C, V)
    o.close()
