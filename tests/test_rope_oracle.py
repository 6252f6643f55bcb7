"""Pins of the oracle's rotary position embedding (RoFormer, named in "GPT-2 from
scratch with torch", token and position embedding, as the newer alternative to the
learned position vectors): closed forms of the rotation, its group properties, the
relative-position property of rotated dot products, the model's wiring of it, and
central finite differences through a whole rotary model."""
import numpy as np
import pytest

import synth
from synth import ModelShape, Workload

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _o():
    import oracle
    return oracle


def test_two_dimensional_case_is_a_plain_rotation_by_the_position():
    # hs = 2: theta_0 = base^0 = 1, so position m turns (x, y) by m radians
    rng = np.random.default_rng(0)
    x = rng.standard_normal((6, 2))
    pos = np.array([0, 1, 2, 5, 100, 1023])
    y = _o().rope(x, pos, base=10000.0)
    c, s = np.cos(pos), np.sin(pos)
    np.testing.assert_allclose(y[:, 0], x[:, 0] * c - x[:, 1] * s, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[:, 1], x[:, 0] * s + x[:, 1] * c, rtol=0, atol=1e-14)


def test_frequencies_fall_geometrically_across_the_pairs():
    # hs = 8, base 10^4: pair i turns by m 10^(-i): pair 3 at m = 1000 by exactly 1 rad,
    # pair 0 at m = 1 by 1 rad; a unit vector on one pair shows the angle directly
    e = np.zeros((2, 8))
    e[0, 6] = 1.0   # pair 3
    e[1, 0] = 1.0   # pair 0
    y = _o().rope(e, np.array([1000, 1]), base=10000.0)
    np.testing.assert_allclose(y[0, 6:8], [np.cos(1.0), np.sin(1.0)], atol=1e-12)
    np.testing.assert_allclose(y[1, 0:2], [np.cos(1.0), np.sin(1.0)], atol=1e-14)
    # the other pairs of those vectors stay zero
    assert not y[0, :6].any() and not y[1, 2:].any()


def test_position_zero_is_the_identity_and_norms_are_kept():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((16, 64))
    np.testing.assert_array_equal(_o().rope(x, np.zeros(16)), x)
    y = _o().rope(x, rng.integers(0, 2048, 16))
    np.testing.assert_allclose(np.linalg.norm(y.reshape(16, 32, 2), axis=2),
                               np.linalg.norm(x.reshape(16, 32, 2), axis=2), rtol=1e-13)


def test_turns_compose_and_invert():
    O = _o()
    rng = np.random.default_rng(2)
    x = rng.standard_normal((10, 32))
    a, b = rng.integers(0, 500, 10), rng.integers(0, 500, 10)
    np.testing.assert_allclose(O.rope(O.rope(x, a), b), O.rope(x, a + b), atol=1e-12)
    np.testing.assert_allclose(O.rope(O.rope(x, a), a, inverse=True), x, atol=1e-13)


def test_rotated_scores_depend_only_on_the_relative_position():
    # <R(m) q, R(n) k> = <R(m - n) q, k>: the property the embedding exists for
    O = _o()
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((1, 64)), rng.standard_normal((1, 64))
    for m, n in [(5, 2), (700, 3), (1023, 1000), (17, 17)]:
        lhs = (O.rope(q, [m]) @ O.rope(k, [n]).T).item()
        rhs = (O.rope(q, [m - n]) @ k.T).item()
        assert lhs == pytest.approx(rhs, abs=1e-11)
        shifted = (O.rope(q, [m + 40]) @ O.rope(k, [n + 40]).T).item()
        assert shifted == pytest.approx(lhs, abs=1e-11)


def _rotary_model(seed=4, NH=2, C=32, T=12):
    from parity_util import rand_params
    w = Workload("rope", ModelShape(16, 29, 2, NH, C), 2, T, "fp32", "uniform", index=60)
    O = _o()
    p = rand_params(w.model, seed=seed)
    o = O.Oracle(w.model, w.B, w.T, "f64")
    o.set("params", p)
    o.set_rotary(True)
    return w, o, p


def test_model_rotates_q_and_k_of_every_head_and_ignores_wpe():
    O = _o()
    w, o, p = _rotary_model(NH=4, C=32)
    x, y = synth.inputs_targets(w)
    loss = o.forward(x, y)
    m = w.model
    C, NH, hs = m.channels, m.num_heads, m.channels // m.num_heads
    for l in range(m.num_layers):
        qkv = o.act("qkv", l).reshape(w.B, w.T, 3 * C)
        rot = o.act("qkv_rot", l).reshape(w.B, w.T, 3 * C)
        pos = np.broadcast_to(np.arange(w.T)[None, :, None], (w.B, w.T, 2 * NH)).reshape(-1)
        heads = qkv[:, :, :2 * C].reshape(-1, hs)
        np.testing.assert_allclose(rot[:, :, :2 * C].reshape(-1, hs), O.rope(heads, pos), atol=1e-13)
        np.testing.assert_array_equal(rot[:, :, 2 * C:], qkv[:, :, 2 * C:])
    # wpe takes no part: other wpe values give the same loss, and its gradient is zero
    off, n = synth.param_offsets(m)["wpe"]
    p2 = p.copy()
    p2[off:off + n] = np.random.default_rng(9).standard_normal(n)
    o.set("params", p2)
    assert o.forward(x, y) == loss
    o.backward()
    assert not o.get("grads")[off:off + n].any()
    # and switching it off gives back the learned-position model
    o.set_rotary(False)
    ref = O.Oracle(m, w.B, w.T, "f64")
    ref.set("params", p2)
    assert o.forward(x, y) == ref.forward(x, y)


def test_single_position_rotary_equals_learned_model_with_zero_position_row():
    # at T = 1 every position is 0, where the turn is the identity
    O = _o()
    w, o, p = _rotary_model(T=1)
    x, y = synth.inputs_targets(w)
    off, n = synth.param_offsets(w.model)["wpe"]
    p0 = p.copy()
    p0[off:off + n] = 0.0
    ref = O.Oracle(w.model, w.B, 1, "f64")
    ref.set("params", p0)
    assert o.forward(x, y) == pytest.approx(ref.forward(x, y), abs=1e-15)


def test_rotary_backward_matches_central_finite_differences():
    # the tiny char-level model, parameters and step of the learned-position
    # finite-difference pin, with the rotary embedding switched on
    from test_oracle_pins import rand_params
    w = synth.WORKLOADS["tiny_char_b4t32_fp32"]
    m = w.model
    p = rand_params(m)
    o = _o().Oracle(m, w.B, w.T, "f64")
    o.set("params", p)
    o.set_rotary(True)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    o.backward()
    g = o.get("grads")
    rng = np.random.default_rng(3)
    h = 1e-5
    for name, (off, n) in synth.param_offsets(m).items():
        if name == "wpe":
            continue
        idx = rng.choice(n, size=min(16, n), replace=False) + off
        if name == "wte":   # ids that occur in the batch
            idx[:4] = off + int(x[0, 0]) * m.channels + np.arange(4)
        for i in idx:
            pp = p.copy(); pp[i] += h
            o.set("params", pp); lp = o.forward(x, y)
            pp[i] -= 2 * h
            o.set("params", pp); lm = o.forward(x, y)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[i]) <= 1e-6 * abs(g[i]) + 1e-9, (name, i, fd, g[i])
