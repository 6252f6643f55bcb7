"""The Llama-style block on the GPU path (through the C ABI) against the oracle's
Llama-style block: RMSNorm, bias-free products, SwiGLU MLP, rotary positions.
fp32 steps are checked tensor by tensor (activations, loss, every gradient, AdamW),
bf16 steps by loss and gradient direction, and the block's refusals are checked."""
import numpy as np
import pytest

import synth
from synth import ModelShape, Workload
from parity_util import BF16_GRAD_COS, cosine, gpu_arena, oracle_model, per_tensor, rand_params, report, to_np
from test_gpu_parity import announce, bf16_compare, fp32_full_compare

pytestmark = pytest.mark.gpu


def llama_params(m, seed):
    """The init recipe plus random RMSNorm gains (the block has no biases)."""
    p = synth.init_params(m).astype(np.float64)
    rng = np.random.default_rng(seed)
    for name, (o, n) in synth.param_offsets(m).items():
        if "rms" in name:
            p[o:o + n] = 1.0 + 0.1 * rng.standard_normal(n)
    return p.astype(np.float32)


@pytest.mark.parametrize("NH,T", [(4, 77), (2, 64), (1, 33)])
def test_fp32_llama_step(NH, T):
    w = Workload("llama_fp32", ModelShape(96, 301, 2, NH, 128, "llama"), 2, T, "fp32", "uniform", index=71)
    announce(f"llama_fp32_hs{128 // NH}_T{T}", w)
    from transformer_lm_fwd_amd import binding as b
    a, o = fp32_full_compare(w, llama_params(w.model, 71 + NH), rotary=True)
    g = to_np(a.tensor(b.T_GRADS)).ravel()
    off, n = synth.param_offsets(w.model)["wpe"]
    assert not g[off:off + n].any()


@pytest.mark.parametrize("T", [64, 130])
def test_bf16_llama_step(T):
    w = Workload("llama_bf16", ModelShape(256, 301, 2, 2, 128, "llama"), 2, T, "bf16", "zipf", index=72)
    announce(f"llama_bf16_T{T}", w)
    bf16_compare(w, llama_params(w.model, 72), rotary=True)


def test_llama_124m_shape_bf16_step_against_the_float_oracle():
    # the 124M-sized Llama-style model (C 768, 12 layers, SwiGLU width 2048) on a short batch
    from transformer_lm_fwd_amd import binding as b
    w = Workload("llama_124m", synth.LLAMA_124M, 2, 64, "bf16", "uniform", index=73)
    announce("llama_124m_b2t64", w)
    params = synth.init_params(w.model)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, params)
    a.forward(x, y)
    loss = a.loss()
    a.backward()
    o = oracle_model(w, params, prec="f32")
    ref = o.forward(x, y)
    o.backward()
    g, gr = to_np(a.tensor(b.T_GRADS)).ravel(), o.get("grads")
    cos = cosine(g, gr)
    cos_t = {k: cosine(v, per_tensor(gr, w.model)[k]) for k, v in per_tensor(g, w.model).items()
             if np.abs(per_tensor(gr, w.model)[k]).max() > 0}
    report("per-tensor cosine", cos_t)
    print(f"loss gpu={loss:.6f} oracle={ref:.6f}; flat gradient cosine {cos:.6f}", flush=True)
    assert abs(loss - ref) <= 2e-2 and cos >= BF16_GRAD_COS


def test_llama_refusals():
    from transformer_lm_fwd_amd import Generator, binding as b
    w = Workload("llama_refuse", ModelShape(64, 97, 1, 2, 128, "llama"), 1, 16, "bf16", "uniform", index=74)
    announce("llama_refusals", w)
    a = gpu_arena(w, llama_params(w.model, 74))
    for call in (lambda: a.set_gemm_format(b.GPT2_GEMM_MXFP8), lambda: a.set_position_encoding(b.GPT2_POS_LEARNED),
                 lambda: Generator(a, 1, 16)):
        with pytest.raises(b.Gpt2Error):
            call()
    with pytest.raises(ValueError):
        a.save_checkpoint("/tmp/never_written.bin", 0)


def test_fp32_llama_single_position():
    w = Workload("llama_t1", ModelShape(16, 97, 2, 2, 64, "llama"), 3, 1, "fp32", "uniform", index=75)
    announce("llama_fp32_T1", w)
    fp32_full_compare(w, llama_params(w.model, 75), rotary=True)
