"""Rotary position embedding on the GPU path (through the C ABI) against the oracle
with the same embedding: forward activations (the qkv rows hold the turned q and k),
loss, every gradient (wpe's is zero), one AdamW step; bf16 at head size 64; the
cached generation path; and the switch back to learned positions."""
import numpy as np
import pytest

import synth
from synth import ModelShape, Workload
from parity_util import cosine, gpu_arena, oracle_model, rand_params, to_np
from test_gpu_parity import announce, bf16_compare, fp32_full_compare

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("NH", [8, 4, 2, 1])
def test_fp32_rotary_step(NH):
    # head sizes 16, 32, 64, 128; a ragged T
    w = Workload("rope_fp32", ModelShape(96, 301, 2, NH, 128), 2, 77, "fp32", "uniform", index=61)
    announce(f"rope_fp32_hs{128 // NH}", w)
    from transformer_lm_fwd_amd import binding as b
    a, o = fp32_full_compare(w, rand_params(w.model, seed=61 + NH), rotary=True)
    off, n = synth.param_offsets(w.model)["wpe"]
    # the AdamW step ran after the gradients were taken; the wpe gradient is still there
    assert not to_np(a.tensor(b.T_GRADS)).ravel()[off:off + n].any()


@pytest.mark.parametrize("T", [64, 200])
def test_bf16_rotary_step(T):
    w = Workload("rope_bf16", ModelShape(256, 301, 2, 2, 128), 2, T, "bf16", "zipf", index=62)
    announce(f"rope_bf16_T{T}", w)
    bf16_compare(w, rand_params(w.model, seed=62), rotary=True)


def test_rotary_changes_the_model_and_switching_back_restores_it():
    from transformer_lm_fwd_amd import binding as b
    w = Workload("rope_switch", ModelShape(96, 301, 2, 2, 128), 2, 40, "bf16", "uniform", index=63)
    announce("rope_switch", w)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, rand_params(w.model, seed=63))
    a.forward(x)
    z0 = to_np(a.tensor(b.T_LOGITS)).copy()
    a.set_position_encoding(b.GPT2_POS_ROTARY)
    a.forward(x)
    z1 = to_np(a.tensor(b.T_LOGITS)).copy()
    assert np.abs(z1 - z0).max() > 1e-3
    # position 0 is turned by zero: its rows depend only on token 0 of each sequence
    # and carry no position vector either way once wpe row 0 is zero
    a.set_position_encoding(b.GPT2_POS_LEARNED)
    a.forward(x)
    np.testing.assert_array_equal(to_np(a.tensor(b.T_LOGITS)), z0)
    with pytest.raises(b.Gpt2Error):
        a.set_position_encoding(b.GPT2_POS_ROTARY, base=1.0)
    with pytest.raises(b.Gpt2Error):
        a.set_position_encoding(7)


def test_rotary_generation_matches_the_oracle_forward():
    from transformer_lm_fwd_amd import Generator
    m = ModelShape(256, 301, 2, 2, 128)
    batch, n, steps = 3, 11, 9
    w = Workload("rope_gen", m, batch, 32, "bf16", "uniform", index=64)
    announce("rope_generation", w, B=batch, T=n + steps)
    from transformer_lm_fwd_amd import binding as b
    params = rand_params(m, seed=64)
    a = gpu_arena(w, params, B=batch, T=n + steps)
    a.set_position_encoding(b.GPT2_POS_ROTARY)
    gen = Generator(a, batch, n + steps)
    seq = synth.token_windows(w, seed=5, B=batch, T=n)[:, :n]
    got = [to_np(gen.prefill(seq)).copy()]
    for _ in range(steps - 1):
        nxt = got[-1].argmax(1).astype(np.int32)
        seq = np.concatenate([seq, nxt[:, None]], 1)
        got.append(to_np(gen.decode(nxt)).copy())
    o = oracle_model(w, params, B=batch, T=seq.shape[1])
    o.set_rotary(True)
    o.forward(seq)
    ref = o.act("logits").reshape(batch, seq.shape[1], -1)
    for i, g in enumerate(got):
        pos = n - 1 + i
        err = np.abs(g - ref[:, pos]).max()
        cos = min(cosine(g[r], ref[r, pos]) for r in range(batch))
        print(f"position {pos}: max |logit - oracle| = {err:.3g}, min row cosine {cos:.6f}", flush=True)
        assert err <= 6e-2 and cos >= 0.9995
