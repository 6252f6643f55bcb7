"""Pins of the oracle's Llama-style block (the layers [llm.c] lists for Llama-2-type
models: RMSNorm, SwiGLU, rotary positions, no biases): its parameter count, the
closed forms of silu, RMSNorm's row statistics, the wiring of the SwiGLU MLP and of
the bias-free products, and central finite differences through the whole model."""
import math

import numpy as np
import pytest

import synth
from synth import ModelShape, Workload

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _o():
    import oracle
    return oracle


TINY = ModelShape(16, 29, 2, 2, 32, "llama")


def test_parameter_count_closed_form():
    O = _o()
    assert synth.llama_hidden(768) == 2048 and synth.llama_hidden(128) == 384 and synth.llama_hidden(32) == 128
    for m in (synth.LLAMA_124M, TINY, ModelShape(64, 97, 3, 4, 96, "llama")):
        C, L, H = m.channels, m.num_layers, synth.llama_hidden(m.channels)
        n = m.vocab_size * C + m.max_seq_len * C + L * (2 * C + 4 * C * C + 3 * H * C) + C
        assert O.num_parameters(m) == n == synth.num_parameters(m)
    # 50257*768 + 1024*768 + 12 * (2*768 + 4*768^2 + 3*2048*768) + 768
    assert O.num_parameters(synth.LLAMA_124M) == 124_337_664


def test_silu_closed_forms():
    O = _o()
    l3 = math.log(3.0)   # sigmoid(ln 3) = 3/4
    x = np.array([0.0, l3, -l3, 40.0, -40.0])
    y = O.silu(x)
    np.testing.assert_allclose(y, [0.0, 0.75 * l3, -0.25 * l3, 40.0, 0.0], atol=1e-15)
    r = np.random.default_rng(0).standard_normal(100) * 4
    np.testing.assert_allclose(O.silu(r) - O.silu(-r), r, atol=1e-14)   # sigmoid(x) + sigmoid(-x) = 1
    assert O.silu_grad(np.array([0.0]))[0] == 0.5
    h = 1e-6
    np.testing.assert_allclose(O.silu_grad(r), (O.silu(r + h) - O.silu(r - h)) / (2 * h), atol=1e-8)


def _model(m, B=2, T=12, seed=3):
    from test_oracle_pins import rand_params
    w = Workload("llama", m, B, T, "fp32", "uniform", index=70)
    p = rand_params(m, seed=seed)
    o = _o().Oracle(m, B, T, "f64")
    o.set("params", p)
    return w, o, p


def test_rmsnorm_rows_and_bias_free_products():
    w, o, p = _model(TINY)
    m = w.model
    offs = synth.param_offsets(m)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    C, BT = m.channels, w.B * w.T
    enc = o.act("encoded").reshape(BT, C)
    ln1 = o.act("ln1", 0).reshape(BT, C)
    g = p[offs["h0.rms1.w"][0]:][:C]
    ms = (enc ** 2).mean(1)
    np.testing.assert_allclose(o.act("ln1_rstd", 0), 1 / np.sqrt(ms + 1e-5), rtol=1e-13)
    assert not o.act("ln1_mean", 0).any()
    # dividing out the gains leaves rows whose mean square is ms / (ms + eps)
    np.testing.assert_allclose(((ln1 / g) ** 2).mean(1), ms / (ms + 1e-5), rtol=1e-12)
    # qkv = ln1 W^T, with no bias (numpy's product)
    W = p[offs["h0.qkv.w"][0]:][:3 * C * C].reshape(3 * C, C)
    np.testing.assert_allclose(o.act("qkv", 0).reshape(BT, 3 * C), ln1 @ W.T, rtol=1e-12, atol=1e-14)
    # rotary positions always on: turning them off is refused
    with pytest.raises(ValueError):
        o.set_rotary(False)


def test_swiglu_wiring():
    O = _o()
    w, o, p = _model(TINY)
    m = w.model
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    H, BT = synth.llama_hidden(m.channels), w.B * w.T
    gu = o.act("fch", 1).reshape(BT, H, 2)
    h = o.act("fch_gelu", 1).reshape(BT, H)
    np.testing.assert_allclose(h, O.silu(gu[:, :, 0]) * gu[:, :, 1], rtol=1e-13, atol=1e-16)
    # the down projection maps h back to C with no bias
    offs = synth.param_offsets(m)
    Wd = p[offs["h1.down.w"][0]:][:m.channels * H].reshape(m.channels, H)
    np.testing.assert_allclose(o.act("residual3", 1) - o.act("residual2", 1),
                               (h @ Wd.T).ravel(), rtol=1e-10, atol=1e-13)


def test_llama_backward_matches_central_finite_differences():
    from test_oracle_pins import rand_params
    m = ModelShape(32, 65, 2, 4, 64, "llama")   # the tiny char model's shape, Llama-style
    w = Workload("llama_fd", m, 4, 32, "fp32", "uniform", index=0)
    p = rand_params(m)
    o = _o().Oracle(m, w.B, w.T, "f64")
    o.set("params", p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    o.backward()
    g = o.get("grads")
    rng = np.random.default_rng(3)
    h = 1e-5
    for name, (off, n) in synth.param_offsets(m).items():
        idx = rng.choice(n, size=min(16, n), replace=False) + off
        if name == "wpe":
            assert not g[off:off + n].any()
            continue
        if name == "wte":
            idx[:4] = off + int(x[0, 0]) * m.channels + np.arange(4)
        for i in idx:
            pp = p.copy(); pp[i] += h
            o.set("params", pp); lp = o.forward(x, y)
            pp[i] -= 2 * h
            o.set("params", pp); lm = o.forward(x, y)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[i]) <= 1e-6 * abs(g[i]) + 1e-9, (name, i, fd, g[i])
