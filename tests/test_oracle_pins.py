"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it rests on (page title, section).  None of them
re-types an oracle formula: they use printed integers, closed forms of special
cases, invariants, independent library routines, central finite differences
and an independent autograd implementation.
"""
import math

import numpy as np
import pytest

import synth
from synth import ModelShape, Workload

pytestmark = pytest.mark.usefixtures("oracle_lib")


def _oracle():
    import oracle
    return oracle


def small_workload(V=65, P=32, L=2, NH=4, C=64, B=4, T=32, tokens="uniform", index=9):
    return Workload("test", ModelShape(P, V, L, NH, C), B, T, "fp32", tokens, index=index)


def rand_params(m, seed=7, scale=1.0):
    """Init recipe plus random LayerNorm gains/shifts and biases, so that no
    term of any gradient is multiplied by an exact 0 or 1."""
    p = synth.init_params(m).astype(np.float64)
    offs = synth.param_offsets(m)
    rng = np.random.default_rng(seed)
    for name, (o, n) in offs.items():
        if name.endswith(("ln1.w", "ln2.w")) or name == "lnf.w":
            p[o:o + n] = 1.0 + 0.1 * rng.standard_normal(n)
        elif name.endswith(".b"):
            p[o:o + n] = 0.1 * rng.standard_normal(n)
    return p * scale


def make(w, params=None, prec="f64", T=None, B=None):
    O = _oracle()
    o = O.Oracle(w.model, w.B if B is None else B, w.T if T is None else T, prec)
    o.set("params", synth.init_params(w.model) if params is None else params)
    return o


# ----------------------------------------------------------------------------- printed integers

def _printed():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pages_printed.json")) as f:
        return json.load(f)


def test_num_parameters_matches_printed_banner():
    # "1000 行 C 代码完成 GPT-2 训练的 LLM.c", 快速开始吧！: the GPT-2 (124M) run banner
    # prints num_parameters 124439808 (tied lm_head, unpadded vocabulary).
    g = _printed()
    m = ModelShape(g["max_seq_len"], g["vocab_size"], g["num_layers"], g["num_heads"], g["channels"])
    assert m == synth.GPT2_124M
    O = _oracle()
    assert O.num_parameters(m) == g["num_parameters"]
    assert synth.num_parameters(m) == g["num_parameters"]


def test_num_activations_matches_printed_banner():
    # Same banner: num_activations 73323776, for the trainer's plain activation set
    # at B*T = 256 tokens (the printed batch counts 1192 and 128 of 305260 and
    # 32768 tokens give B*T = 256; B = 4, T = 64 is the split that fits).
    g = _printed()
    assert g["train_tokens"] // 256 == g["train_num_batches"] and g["val_tokens"] // 256 == g["val_num_batches"]
    O = _oracle()
    assert O.num_activations(synth.GPT2_124M, 4, 64) == g["num_activations"]
    assert O.num_activations(synth.GPT2_124M, 8, 32) != g["num_activations"]


def test_parameter_counts_of_other_shapes_follow_the_same_list():
    O = _oracle()
    for m in (synth.GPT2_TINY_CHAR, synth.GPT2_350M, synth.GPT2_1558M):
        C, L = m.channels, m.num_layers
        # token and position tables, 12 C^2 + 13 C per block, final LayerNorm
        expect = m.vocab_size * C + m.max_seq_len * C + L * (12 * C * C + 13 * C) + 2 * C
        assert O.num_parameters(m) == expect == synth.num_parameters(m)


# ----------------------------------------------------------------------------- cross-entropy

@pytest.mark.parametrize("V", [65, 50257])
def test_zero_logits_give_loss_ln_V(V):
    # "从头搭建GPT(Andrej Karpathy) 笔记", 计算loss: a uniform guess over 65 symbols costs
    # -ln(1/65) ~ 4.17.  With ln_f gain and shift 0 every logit is exactly 0.
    w = small_workload(V=V, P=8, L=1, NH=2, C=16, B=2, T=4)
    p = rand_params(w.model)
    o_lnf_w, n = synth.param_offsets(w.model)["lnf.w"]
    p[o_lnf_w:o_lnf_w + 2 * n] = 0.0
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    loss = o.forward(x, y)
    assert loss == pytest.approx(math.log(V), rel=1e-14)
    o.backward()
    dz = o.act("dlogits").reshape(w.B * w.T, V)
    onehot = np.zeros_like(dz)
    onehot[np.arange(w.B * w.T), y.reshape(-1)] = 1.0
    np.testing.assert_allclose(dz, (1.0 / V - onehot) / (w.B * w.T), rtol=1e-12, atol=1e-18)


def test_softmax_rows_sum_to_one_and_dlogits_rows_sum_to_zero():
    w = small_workload()
    o = make(w, rand_params(w.model))
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    o.backward()
    V = w.model.vocab_size
    probs = o.act("probs").reshape(-1, V)
    np.testing.assert_allclose(probs.sum(1), 1.0, rtol=0, atol=1e-13)
    assert (probs > 0).all()
    dz = o.act("dlogits").reshape(-1, V)
    np.testing.assert_allclose(dz.sum(1), 0.0, atol=1e-16)
    # the loss of each row is -log of the target probability
    losses = o.act("losses")
    np.testing.assert_allclose(losses, -np.log(probs[np.arange(probs.shape[0]), y.reshape(-1)]), rtol=1e-12)


def test_initial_loss_is_close_to_ln_V():
    # 计算loss: near-uniform predictions at initialisation cost about ln V.
    g = _printed()
    assert abs(math.log(g["char_vocab"]) - g["uniform_guess_loss_char_vocab_approx"]) < 0.005
    w = synth.WORKLOADS["tiny_char_b4t32_fp32"]
    assert w.model.vocab_size == g["char_vocab"]
    o = make(w)
    x, y = synth.inputs_targets(w)
    assert abs(o.forward(x, y) - math.log(65)) < 0.5


# ----------------------------------------------------------------------------- attention

def _zero_rows(p, m, layer, rows):
    o, _ = synth.param_offsets(m)[f"h{layer}.qkv.w"]
    ob, _ = synth.param_offsets(m)[f"h{layer}.qkv.b"]
    C = m.channels
    for r0, r1 in rows:
        p[o + r0 * C:o + r1 * C] = 0.0
        p[ob + r0:ob + r1] = 0.0


def test_zero_queries_and_keys_give_prefix_means():
    # "从头搭建GPT(Andrej Karpathy) 笔记", 直觉上的self-attention: with equal scores the
    # lower-triangular mask and softmax average all earlier positions (the tril
    # matrix, row-normalised, times V gives prefix means).
    w = small_workload()
    m = w.model
    p = rand_params(m)
    for l in range(m.num_layers):
        _zero_rows(p, m, l, [(0, 2 * m.channels)])   # q and k rows of c_attn
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    C = m.channels
    for l in range(m.num_layers):
        qkv = o.act("qkv", l).reshape(w.B, w.T, 3 * C)
        v = qkv[:, :, 2 * C:]
        expect = np.cumsum(v, axis=1) / np.arange(1, w.T + 1)[None, :, None]
        np.testing.assert_allclose(o.act("atty", l).reshape(w.B, w.T, C), expect, rtol=1e-12, atol=1e-14)


def test_constant_values_give_ones():
    # Attention weights of every row sum to one: v == 1 makes every output 1.
    w = small_workload()
    m = w.model
    p = rand_params(m)
    C = m.channels
    for l in range(m.num_layers):
        _zero_rows(p, m, l, [(2 * C, 3 * C)])
        ob, _ = synth.param_offsets(m)[f"h{l}.qkv.b"]
        p[ob + 2 * C:ob + 3 * C] = 1.0
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    for l in range(m.num_layers):
        np.testing.assert_allclose(o.act("atty", l), 1.0, rtol=0, atol=1e-14)
        att = o.act("att", l).reshape(w.B, m.num_heads, w.T, w.T)
        np.testing.assert_allclose(att.sum(-1), 1.0, atol=1e-14)
        # masked (future) weights are exactly zero
        iu = np.triu_indices(w.T, 1)
        assert (att[:, :, iu[0], iu[1]] == 0).all()


def test_single_position_attends_to_itself():
    w = small_workload(T=1)
    o = make(w, rand_params(w.model))
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    C = w.model.channels
    for l in range(w.model.num_layers):
        qkv = o.act("qkv", l).reshape(w.B, 3 * C)
        np.testing.assert_array_equal(o.act("atty", l).reshape(w.B, C), qkv[:, 2 * C:])


def test_causality_future_tokens_leave_past_logits_bit_identical():
    # "GPT-2 from scratch with torch", 自注意力: the causal mask lets each position
    # see only itself and earlier positions.
    w = small_workload()
    o = make(w, rand_params(w.model))
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    ref = o.act("logits").reshape(w.B, w.T, -1).copy()
    for t in (0, 5, 17, w.T - 2):
        x2 = x.copy()
        x2[:, t + 1:] = (x2[:, t + 1:] + 7) % w.model.vocab_size
        o.forward(x2, y)
        z = o.act("logits").reshape(w.B, w.T, -1)
        np.testing.assert_array_equal(z[:, :t + 1], ref[:, :t + 1])
        assert not np.array_equal(z[:, t + 1:], ref[:, t + 1:])


def test_prefix_run_reproduces_full_run_rows():
    # Consequence of causality used by the full-size GPU checks: the first t0
    # positions of a length-T run equal a run on the length-t0 prefix.
    w = small_workload()
    p = rand_params(w.model)
    x, y = synth.inputs_targets(w)
    full = make(w, p)
    full.forward(x, y)
    t0 = 11
    pre = make(w, p, T=t0)
    pre.forward(x[:, :t0], y[:, :t0])
    np.testing.assert_array_equal(pre.act("logits").reshape(w.B, t0, -1),
                                  full.act("logits").reshape(w.B, w.T, -1)[:, :t0])
    np.testing.assert_array_equal(pre.act("losses").reshape(w.B, t0),
                                  full.act("losses").reshape(w.B, w.T)[:, :t0])


# ----------------------------------------------------------------------------- embedding, layernorm, linear

def test_encoder_is_a_row_gather_plus_position_rows():
    # "GPT-2 from scratch with torch", token/position embedding: x = wte(tokens) + wpe(positions 0..T-1).
    w = small_workload()
    m = w.model
    p = rand_params(m)
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    C = m.channels
    ow, _ = synth.param_offsets(m)["wte"]
    op, _ = synth.param_offsets(m)["wpe"]
    wte = p[ow:ow + m.vocab_size * C].reshape(m.vocab_size, C)
    wpe = p[op:op + m.max_seq_len * C].reshape(m.max_seq_len, C)
    np.testing.assert_array_equal(o.act("encoded").reshape(w.B, w.T, C), wte[x] + wpe[None, :w.T])


def test_layernorm_output_rows_are_standardised():
    # "GPT-2 from scratch with torch", Transformer block: LayerNorm standardises each
    # position over its channels (eps 1e-5).  With gain 1 and shift 0 each row has
    # mean 0 and variance var/(var + eps), var the row's biased variance.
    w = small_workload()
    o = make(w)            # init recipe: gains 1, shifts 0
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    C = w.model.channels
    xin = o.act("encoded").reshape(-1, C)
    ln = o.act("ln1", 0).reshape(-1, C)
    var = xin.var(axis=1)
    np.testing.assert_allclose(ln.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose(ln.var(axis=1), var / (var + 1e-5), rtol=1e-12)
    np.testing.assert_allclose(o.act("ln1_mean", 0), xin.mean(axis=1), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(o.act("ln1_rstd", 0), 1 / np.sqrt(var + 1e-5), rtol=1e-12)


def test_linear_layers_and_tied_logits_match_numpy_matmul():
    # "GPT-2ベースの3000バイトCで実装されたChatGPTクローン", ニューラルネットワーク層の実装:
    # Linear is a matrix product plus a bias repeated per row; Transformer本体: the
    # logits are the final hidden state times the embedding matrix.
    w = small_workload()
    m = w.model
    p = rand_params(m)
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    C, V = m.channels, m.vocab_size
    offs = synth.param_offsets(m)

    def tensor(name, shape):
        a, n = offs[name]
        return p[a:a + n].reshape(shape)

    ln1 = o.act("ln1", 1).reshape(-1, C)
    np.testing.assert_allclose(o.act("qkv", 1).reshape(-1, 3 * C),
                               ln1 @ tensor("h1.qkv.w", (3 * C, C)).T + tensor("h1.qkv.b", (3 * C,)), rtol=1e-12, atol=1e-13)
    g = o.act("fch_gelu", 0).reshape(-1, 4 * C)
    np.testing.assert_allclose(o.act("fcproj", 0).reshape(-1, C),
                               g @ tensor("h0.fcproj.w", (C, 4 * C)).T + tensor("h0.fcproj.b", (C,)), rtol=1e-12, atol=1e-13)
    lnf = o.act("lnf").reshape(-1, C)
    np.testing.assert_allclose(o.act("logits").reshape(-1, V), lnf @ tensor("wte", (V, C)).T, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- GELU

def test_gelu_tanh_form_identities():
    # "GPT-2ベースの3000バイトCで..." comment thread prints the tanh approximation
    # x/2 (1 + tanh(.7978845 (x + .044715 x^3))); .7978845 is sqrt(2/pi) truncated.
    O = _oracle()
    x = np.linspace(-8, 8, 4001)
    g = O.gelu(x)
    # (1 + tanh(u)) / 2 = logistic(2u): the same function by another route
    u = math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)
    np.testing.assert_allclose(g, x / (1 + np.exp(-2 * u)), rtol=1e-14, atol=1e-15)
    # tanh is odd, so g(x) - g(-x) = x
    np.testing.assert_allclose(g - O.gelu(-x), x, rtol=1e-14, atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0


def test_gelu_is_the_tanh_form_not_the_erf_form():
    # The same comment notes the exact GELU is x * Phi(x); the tanh form differs by
    # at most ~5e-4, so a test can tell them apart.
    O = _oracle()
    x = np.linspace(-6, 6, 2401)
    exact = x * 0.5 * (1 + np.array([math.erf(v / math.sqrt(2)) for v in x]))
    diff = np.abs(O.gelu(x) - exact)
    assert 1e-4 < diff.max() < 1e-3


def test_gelu_derivative_matches_central_differences():
    O = _oracle()
    x = np.linspace(-6, 6, 1201)
    h = 1e-5
    fd = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_grad(x), fd, rtol=1e-8, atol=1e-9)


# ----------------------------------------------------------------------------- AdamW

def test_adamw_first_step_closed_form():
    # "1000 行 C 代码..." : the trainer's update is Adam (lr 1e-4).  From m = v = 0 the
    # bias-corrected first step is -lr * g / (|g| + eps), plus the decoupled decay.
    w = small_workload()
    p = rand_params(w.model)
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    o.backward()
    g = o.get("grads")
    lr, wd, eps = 1e-3, 0.1, 1e-8
    o.adamw(lr, 0.9, 0.999, eps, wd, 1)
    np.testing.assert_allclose(o.get("params"), p - lr * (g / (np.abs(g) + eps) + wd * p), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(o.get("m"), 0.1 * g, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(o.get("v"), 0.001 * g * g, rtol=1e-12, atol=1e-300)


def test_adamw_constant_gradient_moves_by_lr_each_step():
    # With the same gradient every step, the bias-corrected moments equal g and g^2
    # exactly, so each step moves theta by -lr * g / (|g| + eps) (wd = 0).
    w = small_workload()
    p = rand_params(w.model)
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    o.backward()
    g = o.get("grads")
    theta = p.copy()
    for t in range(1, 4):
        o.set("grads", g)
        o.adamw(1e-3, 0.9, 0.999, 1e-8, 0.0, t)
        theta = theta - 1e-3 * g / (np.abs(g) + 1e-8)
        np.testing.assert_allclose(o.get("params"), theta, rtol=1e-10, atol=1e-13)


# ----------------------------------------------------------------------------- gradients

def test_backward_matches_central_finite_differences():
    # Every backward formula, by brute force on the tiny char-level model
    # (V = 65 from 计算loss), in float64.
    w = synth.WORKLOADS["tiny_char_b4t32_fp32"]
    m = w.model
    p = rand_params(m)
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    o.forward(x, y)
    o.backward()
    g = o.get("grads")
    rng = np.random.default_rng(3)
    h = 1e-5
    worst = 0.0
    for name, (off, n) in synth.param_offsets(m).items():
        idx = rng.choice(n, size=min(16, n), replace=False) + off
        if name == "wte":   # make sure ids that occur in the batch are probed
            C = m.channels
            idx[:4] = off + int(x[0, 0]) * C + np.arange(4)
        for i in idx:
            pp = p.copy(); pp[i] += h
            o.set("params", pp); lp = o.forward(x, y)
            pp[i] -= 2 * h
            o.set("params", pp); lm = o.forward(x, y)
            fd = (lp - lm) / (2 * h)
            err = abs(fd - g[i])
            assert err <= 1e-6 * abs(g[i]) + 1e-9, (name, i, fd, g[i])
            worst = max(worst, err)
    assert worst < 1e-8


def test_backward_matches_torch_autograd():
    # An independent implementation of the same forward (torch ops, float64) whose
    # gradients come from autograd.
    torch = pytest.importorskip("torch")
    w = small_workload(index=11)
    m = w.model
    p = rand_params(m, seed=11)
    o = make(w, p)
    x, y = synth.inputs_targets(w)
    loss = o.forward(x, y)
    o.backward()
    g = o.get("grads")

    C, NH, L, V = m.channels, m.num_heads, m.num_layers, m.vocab_size
    B, T = w.B, w.T
    pt = torch.tensor(p, dtype=torch.float64, requires_grad=True)
    offs = synth.param_offsets(m)

    def P(name, *shape):
        a, n = offs[name]
        return pt[a:a + n].view(*shape)

    F = torch.nn.functional
    xt = torch.tensor(x, dtype=torch.long)
    h = P("wte", V, C)[xt] + P("wpe", m.max_seq_len, C)[:T][None]
    mask = torch.ones(T, T, dtype=torch.bool).tril()
    for l in range(L):
        a = F.layer_norm(h, (C,), P(f"h{l}.ln1.w", C), P(f"h{l}.ln1.b", C), eps=1e-5)
        qkv = F.linear(a, P(f"h{l}.qkv.w", 3 * C, C), P(f"h{l}.qkv.b", 3 * C))
        q, k, v = qkv.split(C, dim=-1)
        q, k, v = (t.view(B, T, NH, C // NH).transpose(1, 2) for t in (q, k, v))
        s = (q @ k.transpose(-1, -2)) / math.sqrt(C // NH)
        s = s.masked_fill(~mask, float("-inf")).softmax(-1)
        yat = (s @ v).transpose(1, 2).reshape(B, T, C)
        h = h + F.linear(yat, P(f"h{l}.proj.w", C, C), P(f"h{l}.proj.b", C))
        a2 = F.layer_norm(h, (C,), P(f"h{l}.ln2.w", C), P(f"h{l}.ln2.b", C), eps=1e-5)
        f = F.gelu(F.linear(a2, P(f"h{l}.fc.w", 4 * C, C), P(f"h{l}.fc.b", 4 * C)), approximate="tanh")
        h = h + F.linear(f, P(f"h{l}.fcproj.w", C, 4 * C), P(f"h{l}.fcproj.b", C))
    h = F.layer_norm(h, (C,), P("lnf.w", C), P("lnf.b", C), eps=1e-5)
    z = h @ P("wte", V, C).T
    lt = F.cross_entropy(z.view(-1, V), torch.tensor(y, dtype=torch.long).view(-1))
    lt.backward()
    assert loss == pytest.approx(lt.item(), rel=1e-13)
    np.testing.assert_allclose(g, pt.grad.numpy(), rtol=1e-9, atol=1e-14)


def test_float_build_agrees_with_double_build():
    # The fp32 oracle's own error sits far inside the GPU tolerances.
    w = small_workload(index=12)
    p = rand_params(w.model, seed=12).astype(np.float32)
    x, y = synth.inputs_targets(w)
    res = {}
    for prec in ("f32", "f64"):
        o = make(w, p, prec=prec)
        loss = o.forward(x, y)
        o.backward()
        res[prec] = (loss, o.act("logits"), o.get("grads"))
    assert abs(res["f32"][0] - res["f64"][0]) <= 1e-6 * abs(res["f64"][0])
    for a, b in ((res["f32"][1], res["f64"][1]), (res["f32"][2], res["f64"][2])):
        assert np.abs(a - b).max() <= 1e-4 * np.abs(b).max()


def test_repeated_steps_on_one_batch_decrease_the_loss():
    # "1000 行 C 代码...", 快速开始吧！: the reference run over-fits one batch for 10
    # iterations; on a fixed batch each Adam step lowers the loss.
    w = synth.WORKLOADS["tiny_char_b4t32_fp32"]
    o = make(w)
    x, y = synth.inputs_targets(w)
    losses = [o.step(x, y, w, t) for t in range(1, 11)]
    assert all(b < a for a, b in zip(losses, losses[1:])), losses


def test_results_do_not_depend_on_thread_count():
    import subprocess, sys, os, json
    code = (
        "import sys, json, numpy as np; sys.path.insert(0, %r)\n"
        "import synth, oracle\n"
        "w = synth.WORKLOADS['tiny_char_b4t32_fp32']\n"
        "o = oracle.Oracle(w.model, w.B, w.T)\n"
        "o.set('params', synth.init_params(w.model))\n"
        "x, y = synth.inputs_targets(w)\n"
        "l = o.forward(x, y); o.backward()\n"
        "print(json.dumps([l, float(np.abs(o.get('grads')).sum()), o.get('grads')[::97].tolist()]))\n"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    outs = []
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, check=True)
        outs.append(json.loads(r.stdout.strip().splitlines()[-1]))
    assert outs[0] == outs[1]
