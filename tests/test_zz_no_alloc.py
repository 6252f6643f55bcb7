"""gpt2_gen_decode_noalloc (the decode step with its row buffers in the library's
static device array) against gpt2_gen_decode, through the C ABI: identical logits,
bit for bit, over several steps, then again with a smaller batch and prompt on a new
state (the array keeps the previous call's contents), and the size limit."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _decode_pair(b, a, batch, prompt_len, steps, seed):
    import torch
    lib = b.lib()
    w = synth.Workload("noalloc", a.m, batch, prompt_len + steps, "bf16", "uniform", index=seed)
    toks = synth.token_windows(w, B=batch, T=prompt_len + steps)
    ref = b.Generator(a, batch, prompt_len + steps)
    new = b.Generator(a, batch, prompt_len + steps)
    p = torch.from_numpy(np.ascontiguousarray(toks[:, :prompt_len])).to(torch.int32).cuda()
    r0 = ref.prefill(p).clone()
    n0 = new.prefill(p).clone()
    assert torch.equal(r0, n0)
    for i in range(steps):
        t = torch.from_numpy(np.ascontiguousarray(toks[:, prompt_len + i])).to(torch.int32).cuda()
        rl = ref.decode(t).clone()
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.gpt2_gen_decode_noalloc(new.h, ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(new.logits.data_ptr()), s)
        assert rc == 0, b.lib().gpt2_last_error().decode()
        torch.cuda.synchronize()
        nl = new.logits.clone()
        print(f"batch {batch} prompt {prompt_len} step {i}: max |noalloc - decode| = "
              f"{float((nl - rl).abs().max()):.3g}", flush=True)
        assert torch.equal(nl, rl)
        assert new.length == ref.length == prompt_len + i + 1
    ref.close()
    new.close()


def test_decode_noalloc_matches_decode_twice_then_smaller():
    import torch
    from transformer_lm_fwd_amd import Arena, binding as b
    torch.cuda.set_device(0)
    m = synth.ModelShape(128, 509, 2, 2, 128)  # head size 64
    print("\n[case] noalloc decode: L=2 NH=2 C=128 V=509 batch 8 then 2", flush=True)
    a = Arena(m, 8, 32, "bf16")
    a.load_params(synth.init_params(m))
    _decode_pair(b, a, batch=8, prompt_len=16, steps=3, seed=40)
    _decode_pair(b, a, batch=2, prompt_len=5, steps=2, seed=41)
    a.close()


def test_decode_noalloc_rejects_rows_beyond_the_static_array():
    import torch
    from transformer_lm_fwd_amd import Arena, binding as b
    torch.cuda.set_device(0)
    m = synth.ModelShape(16, 301, 1, 25, 1600)  # head size 64, C = 1600
    print("\n[case] noalloc decode size limit: L=1 NH=25 C=1600 batch 16 (rejected), 12 (accepted)", flush=True)
    a = Arena(m, 16, 4, "bf16")
    a.load_params(synth.init_params(m))
    lib = b.lib()
    for batch, ok in ((16, False), (12, True)):
        g = b.Generator(a, batch, 4)
        tok = torch.zeros(batch, 2, dtype=torch.int32, device="cuda")
        g.prefill(tok)
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = lib.gpt2_gen_decode_noalloc(g.h, ctypes.c_void_p(tok.data_ptr()), ctypes.c_void_p(g.logits.data_ptr()), s)
        torch.cuda.synchronize()
        assert (rc == 0) == ok, (batch, rc, b.lib().gpt2_last_error().decode())
        if not ok:
            assert rc == -2 and "static scratch" in b.lib().gpt2_last_error().decode()
        g.close()
    a.close()
