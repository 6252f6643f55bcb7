"""Incremental generation with a key/value cache, on the GPU through the C ABI.

The next-token logits after a prefix are, by definition, the forward pass's logits at
the prefix's last position ("GPT-2ベースの3000バイトCで実装されたChatGPTクローン",
KVキャッシュ方式: the cache only saves recomputing the earlier rows).  So every logit
row a prefill or decode step returns is compared with the oracle's forward pass over
the same tokens, and with the GPU's own full forward pass."""
import numpy as np
import pytest

import synth
from synth import ModelShape, Workload
from parity_util import cosine, gpu_arena, oracle_model, rand_params, to_np

pytestmark = pytest.mark.gpu

# Logit tolerance for the bf16 path.  Activations are rounded to bf16 (relative
# 2^-9) after every one of the ~6 stages per layer, and the prefill's logits are
# themselves bf16; for the small models here (|logits| <= ~4) that bounds the error by
# a few hundredths.  Cosine per row and the absolute error are both checked.
GEN_LOGIT_ABS = 6e-2
GEN_ROW_COS = 0.9995


def announce(name, m, batch, n, extra=""):
    print(f"\n[case] {name}: L={m.num_layers} NH={m.num_heads} C={m.channels} V={m.vocab_size} "
          f"batch={batch} prompt={n} {extra}", flush=True)


def prompt_tokens(w, batch, n, seed):
    return synth.token_windows(w, seed=seed, B=batch, T=n)[:, :n]


def greedy_run(gen, prompt, steps):
    """prefill + `steps` greedy decode steps; returns the sequences (prompt + the
    `steps` chosen tokens) and the steps + 1 logit blocks, block i being the
    next-token logits at position n - 1 + i."""
    out = [to_np(gen.prefill(prompt)).copy()]
    seq = prompt.copy()
    for _ in range(steps):
        nxt = out[-1].argmax(1).astype(np.int32)
        seq = np.concatenate([seq, nxt[:, None]], 1)
        out.append(to_np(gen.decode(nxt)).copy())
    return seq, out


def oracle_logits(w, params, seq, prec="f64"):
    B, T = seq.shape
    o = oracle_model(w, params, B=B, T=T, prec=prec)
    o.forward(seq)
    return o.act("logits").reshape(B, T, -1)


def compare(got, ref, label):
    err = np.abs(got - ref).max()
    cos = min(cosine(got[r], ref[r]) for r in range(got.shape[0]))
    print(f"{label}: max |logit - oracle| = {err:.3g}, min row cosine = {cos:.6f}", flush=True)
    assert err <= GEN_LOGIT_ABS and cos >= GEN_ROW_COS, label


@pytest.mark.parametrize("batch,n,steps,C", [(3, 17, 12, 128), (1, 1, 20, 128), (16, 5, 4, 128), (8, 6, 5, 64),
                                             (16, 3, 3, 768)])
def test_prefill_and_decode_match_the_oracle_forward(batch, n, steps, C):
    # C = 64: products with fewer 32-k steps than waves; C = 128 and 768: split-K products
    from transformer_lm_fwd_amd import Generator
    m = ModelShape(256, 301, 2, C // 64, C)  # head size 64
    w = Workload("gen_small", m, batch, 32, "bf16", "uniform", index=31)
    announce("gen_small", m, batch, n, f"steps={steps}")
    params = rand_params(m, seed=31)
    a = gpu_arena(w, params, B=batch, T=max(n, 8))
    gen = Generator(a, batch, n + steps)
    seq, got = greedy_run(gen, prompt_tokens(w, batch, n, seed=100 + n), steps)
    assert gen.length == n + steps
    ref = oracle_logits(w, params, seq)  # got[i] is position n - 1 + i, the last one included
    for i, g in enumerate(got):
        compare(g, ref[:, n - 1 + i, :], f"position {n - 1 + i}")
    # every greedy choice is (within the tolerance) a maximum of the oracle's logits
    for i in range(steps):
        pos = n - 1 + i
        chosen = ref[np.arange(batch), pos, seq[:, n + i]]
        assert np.all(chosen >= ref[:, pos, :].max(1) - 2 * GEN_LOGIT_ABS)


@pytest.mark.parametrize("n,steps", [(250, 12), (500, 30)])
def test_decode_over_long_contexts_matches_the_oracle_forward(n, steps):
    # hundreds of cached keys: every wave of the decode attention takes several 64-key
    # chunks, the last one ragged, and its online softmax rescales across them
    from transformer_lm_fwd_amd import Generator
    m = ModelShape(1024, 301, 2, 2, 128)
    batch = 3
    w = Workload("gen_small", m, batch, n + steps, "bf16", "uniform", index=35)
    announce("gen_long", m, batch, n, f"steps={steps}")
    params = rand_params(m, seed=35)
    a = gpu_arena(w, params, B=batch, T=n)
    gen = Generator(a, batch, n + steps)
    seq, got = greedy_run(gen, prompt_tokens(w, batch, n, seed=200 + n), steps)
    ref = oracle_logits(w, params, seq)
    for i, g in enumerate(got):
        compare(g, ref[:, n - 1 + i, :], f"position {n - 1 + i}")


@pytest.mark.parametrize("batch", [1, 16])
def test_decode_with_a_wide_vocabulary(batch):
    # an lm_head of 20011 columns: 1251 blocks of 16 columns, the last one ragged, at one
    # and at the largest number of rows the skinny product takes
    from transformer_lm_fwd_amd import Generator
    m = ModelShape(64, 20011, 1, 2, 128)
    n, steps = 5, 3
    w = Workload("gen_wide", m, batch, n + steps, "bf16", "uniform", index=36)
    announce("gen_wide_vocab", m, batch, n, f"steps={steps}")
    params = rand_params(m, seed=36)
    a = gpu_arena(w, params, B=batch, T=n)
    gen = Generator(a, batch, n + steps)
    seq, got = greedy_run(gen, prompt_tokens(w, batch, n, seed=300 + batch), steps)
    ref = oracle_logits(w, params, seq)
    for i, g in enumerate(got):
        compare(g, ref[:, n - 1 + i, :], f"position {n - 1 + i}")


def test_decode_matches_the_gpu_full_forward_and_stops_at_max_len():
    from transformer_lm_fwd_amd import Generator, Gpt2Error
    m = ModelShape(256, 301, 2, 2, 128)
    batch, n, steps = 4, 9, 7
    w = Workload("gen_small", m, batch, n + steps, "bf16", "uniform", index=32)
    announce("gen_vs_forward", m, batch, n, f"steps={steps}")
    params = rand_params(m, seed=32)
    a = gpu_arena(w, params, B=batch, T=n + steps)
    gen = Generator(a, batch, n + steps)
    seq, got = greedy_run(gen, prompt_tokens(w, batch, n, seed=7), steps)
    with pytest.raises(Gpt2Error) as e:   # the cache is full
        gen.decode(np.zeros(batch, np.int32))
    assert e.value.code == -2
    # the same arena's training forward over the whole sequence (this clobbers the
    # prefill's activations, which the cache no longer needs)
    full = seq.astype(np.int32)
    a.forward(full)
    from transformer_lm_fwd_amd import binding
    z = to_np(a.tensor(binding.T_LOGITS)).reshape(batch, n + steps, -1)
    for i, g in enumerate(got):
        compare(g, z[:, n - 1 + i, :], f"vs GPU forward, position {n - 1 + i}")


def test_a_second_prefill_restarts_the_cache():
    from transformer_lm_fwd_amd import Generator
    m = ModelShape(256, 301, 2, 2, 128)
    w = Workload("gen_small", m, 2, 16, "bf16", "uniform", index=33)
    announce("gen_restart", m, 2, 6)
    params = rand_params(m, seed=33)
    a = gpu_arena(w, params, B=2, T=16)
    gen = Generator(a, 2, 16)
    p1, p2 = prompt_tokens(w, 2, 6, seed=1), prompt_tokens(w, 2, 6, seed=2)
    _, first = greedy_run(gen, p1, 3)
    _, other = greedy_run(gen, p2, 3)
    _, again = greedy_run(gen, p1, 3)
    assert gen.length == 9
    for x, y in zip(first, again):
        np.testing.assert_array_equal(x, y)   # same kernels, same order: bitwise
    assert any(np.abs(x - y).max() > 0 for x, y in zip(first, other))


def test_sampling_from_decode_logits_stays_in_the_top_k():
    from transformer_lm_fwd_amd import Generator, sample_topk
    import oracle
    m = ModelShape(256, 301, 2, 2, 128)
    batch, n, k = 3, 5, 10
    w = Workload("gen_small", m, batch, 16, "bf16", "uniform", index=34)
    announce("gen_sample", m, batch, n, f"top-{k}")
    a = gpu_arena(w, rand_params(m, seed=34), B=batch, T=16)
    gen = Generator(a, batch, 16)
    logits = to_np(gen.prefill(prompt_tokens(w, batch, n, seed=3)))
    for step in range(6):
        u = synth.uniform53(900 + step, np.arange(batch, dtype=np.uint64)).astype(np.float32)
        tok = sample_topk(logits, k, 0.9, u)
        for r in range(batch):
            assert tok[r] == oracle.sample_topk(logits[r], k, 0.9, u[r])
            assert tok[r] in np.argsort(-logits[r], kind="stable")[:k]
        logits = to_np(gen.decode(tok))


def test_gpt2_124m_batch8_prefill_and_decode_against_the_oracle():
    from transformer_lm_fwd_amd import Generator
    w = synth.WORKLOADS["gpt2_124m_b8t1024_bf16"]
    batch, n, steps = 8, 64, 4
    announce("gen_124m", w.model, batch, n, f"steps={steps}")
    params = synth.init_params(w.model)
    a = gpu_arena(w, params, B=batch, T=n)
    gen = Generator(a, batch, 128)
    seq, got = greedy_run(gen, prompt_tokens(w, batch, n, seed=124), steps)
    ref = oracle_logits(w, params, seq, prec="f32")
    for i, g in enumerate(got):
        compare(g, ref[:, n - 1 + i, :], f"124M position {n - 1 + i}")
