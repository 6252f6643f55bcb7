"""Host-side checks of the C ABI: exported symbols, layout queries and argument
validation.  No kernel runs here (size queries and rejected arguments never
touch the GPU), so these run without a GPU."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from transformer_lm_fwd_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from transformer_lm_fwd_amd import build
        build.build()
    return binding


def declared_functions():
    src = open(os.path.join(ROOT, "include", "gpt2.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(gpt2_\w+)\s*\(", src, re.M)))


def test_header_declares_the_four_step_entry_points():
    names = declared_functions()
    for n in ("gpt2_alloc_arena", "gpt2_forward", "gpt2_backward", "gpt2_adamw_step"):
        assert n in names


def test_library_exports_every_declared_symbol():
    b = _lib()
    L = ctypes.CDLL(b.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(b.EXPORTS)


def test_num_parameters_matches_generator_layout():
    b = _lib()
    for m in (synth.GPT2_TINY_CHAR, synth.GPT2_124M, synth.GPT2_350M, synth.GPT2_1558M):
        assert b.num_parameters(m) == synth.num_parameters(m)
    assert b.num_parameters(synth.GPT2_124M) == 124439808


def test_arena_size_query_and_monotonicity():
    b = _lib()
    m = synth.GPT2_124M
    fp32 = b.arena_bytes(m, 4, 64, b.GPT2_FP32)
    bf16 = b.arena_bytes(m, 4, 64, b.GPT2_BF16)
    assert fp32 > 4 * 4 * 124439808 and bf16 > 0
    assert b.arena_bytes(m, 8, 1024, b.GPT2_BF16) > bf16
    # every workload fits a 288 GB device with room to spare
    for w in synth.WORKLOADS.values():
        dt = b.GPT2_BF16 if w.dtype == "bf16" else b.GPT2_FP32
        assert b.arena_bytes(w.model, w.B, w.T, dt) < 64e9


@pytest.mark.parametrize("shape,B,T,dtype,msg", [
    ((1024, 50257, 12, 12, 770), 4, 64, 0, "multiple of num_heads"),
    ((1024, 50257, 12, 5, 760), 4, 64, 0, "head size"),
    ((64, 65, 2, 4, 64), 4, 65, 0, "max_seq_len"),
    ((64, 65, 2, 4, 64), 0, 8, 0, "B >= 1"),
    ((64, 65, 2, 4, 64), 2, 8, 7, "dtype"),
    ((64, 1, 2, 4, 64), 2, 8, 0, "non-positive"),
])
def test_invalid_configurations_are_rejected(shape, B, T, dtype, msg):
    b = _lib()
    cfg = b.gpt2_config(*shape)
    need = ctypes.c_size_t(0)
    rc = b.lib().gpt2_alloc_arena(ctypes.byref(cfg), B, T, dtype, None, 0, ctypes.byref(need), None)
    assert rc == -1
    assert msg in b.lib().gpt2_last_error().decode()


def test_small_or_misaligned_buffers_are_rejected_without_touching_memory():
    b = _lib()
    cfg = b.make_config(synth.GPT2_TINY_CHAR)
    need = b.arena_bytes(synth.GPT2_TINY_CHAR, 4, 32, b.GPT2_FP32)
    h = ctypes.c_void_p()
    # a fake, never dereferenced address: validation fails before any use
    rc = b.lib().gpt2_alloc_arena(ctypes.byref(cfg), 4, 32, 0, ctypes.c_void_p(1 << 40), need - 1, None, ctypes.byref(h))
    assert rc == -2 and not h.value
    rc = b.lib().gpt2_alloc_arena(ctypes.byref(cfg), 4, 32, 0, ctypes.c_void_p((1 << 40) + 16), need, None, ctypes.byref(h))
    assert rc == -3 and not h.value


def test_backward_before_forward_is_a_state_error_and_step_must_be_positive():
    b = _lib()
    cfg = b.make_config(synth.GPT2_TINY_CHAR)
    need = b.arena_bytes(synth.GPT2_TINY_CHAR, 4, 32, b.GPT2_FP32)
    h = ctypes.c_void_p()
    # a handle over a fake address: only calls that fail validation are made with it
    assert b.lib().gpt2_alloc_arena(ctypes.byref(cfg), 4, 32, 0, ctypes.c_void_p(1 << 40), need, None, ctypes.byref(h)) == 0
    try:
        assert b.lib().gpt2_backward(h, None) == -4
        assert b.lib().gpt2_adamw_step(h, 1e-4, 0.9, 0.999, 1e-8, 0.0, 0, None) == -1
        assert b.lib().gpt2_backward_adamw(h, 1e-4, 0.9, 0.999, 1e-8, 0.0, 0, None) == -1   # step < 1
        assert b.lib().gpt2_backward_adamw(h, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1, None) == -4   # no loss forward
        off, rows, cols, ld, dt = (ctypes.c_size_t(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(),
                                   ctypes.c_int32())
        assert b.lib().gpt2_tensor_info(h, 8, 0, ctypes.byref(off), ctypes.byref(rows), ctypes.byref(cols),
                                        ctypes.byref(ld), ctypes.byref(dt)) == 0
        assert (rows.value, cols.value, ld.value) == (4 * 32, 65, 128) and off.value % 256 == 0
        assert b.lib().gpt2_tensor_info(h, 18, 2, None, None, None, None, None) == -1   # layer out of range
        assert b.lib().gpt2_tensor_info(h, 4, 0, None, None, None, None, None) == -1    # no bf16 copy in fp32
        assert b.lib().gpt2_tensor_info(h, 99, 0, None, None, None, None, None) == -1
    finally:
        b.lib().gpt2_free_arena(h)


def test_binding_refuses_out_of_range_token_ids_on_the_host():
    b = _lib()
    a = b.Arena.__new__(b.Arena)   # no device memory: only the host-side id check is exercised
    a.m, a.B, a.T = synth.GPT2_TINY_CHAR, 2, 3
    import numpy as np
    with pytest.raises(ValueError):
        a._ids(np.array([[0, 1, 65], [0, 0, 0]]))
    with pytest.raises(ValueError):
        a._ids(np.array([[0, 1, -1], [0, 0, 0]]))
    with pytest.raises(ValueError):
        a._ids(np.zeros((3, 2), dtype=np.int32))


def test_generation_state_validation_without_touching_memory():
    b = _lib()
    shape64 = synth.ModelShape(256, 301, 2, 2, 128)   # head size 64
    h = ctypes.c_void_p()
    need = ctypes.c_size_t()
    lib = b.lib()
    # fp32 arena: generation is refused
    cfg = b.make_config(shape64)
    n32 = b.arena_bytes(shape64, 2, 64, b.GPT2_FP32)
    assert lib.gpt2_alloc_arena(ctypes.byref(cfg), 2, 64, 0, ctypes.c_void_p(1 << 40), n32, None, ctypes.byref(h)) == 0
    try:
        assert lib.gpt2_gen_alloc(h, 2, 64, None, 0, ctypes.byref(need), None) == -1
    finally:
        lib.gpt2_free_arena(h)
    # bf16 arena with head size 16: refused
    cfg16 = b.make_config(synth.GPT2_TINY_CHAR)
    n16 = b.arena_bytes(synth.GPT2_TINY_CHAR, 2, 32, b.GPT2_BF16)
    assert lib.gpt2_alloc_arena(ctypes.byref(cfg16), 2, 32, 1, ctypes.c_void_p(1 << 40), n16, None, ctypes.byref(h)) == 0
    try:
        assert lib.gpt2_gen_alloc(h, 1, 8, None, 0, ctypes.byref(need), None) == -1
    finally:
        lib.gpt2_free_arena(h)
    nb = b.arena_bytes(shape64, 2, 64, b.GPT2_BF16)
    assert lib.gpt2_alloc_arena(ctypes.byref(cfg), 2, 64, 1, ctypes.c_void_p(1 << 40), nb, None, ctypes.byref(h)) == 0
    try:
        assert lib.gpt2_gen_alloc(None, 2, 64, None, 0, ctypes.byref(need), None) == -1
        for batch, max_len in [(0, 8), (17, 8), (2, 0), (2, 257)]:
            assert lib.gpt2_gen_alloc(h, batch, max_len, None, 0, ctypes.byref(need), None) == -1, (batch, max_len)
        # size query: the cache ([L][batch][max_len][3C] bf16) dominates and grows with both
        assert lib.gpt2_gen_alloc(h, 2, 64, None, 0, ctypes.byref(need), None) == 0
        n1 = need.value
        assert n1 >= 2 * 2 * 64 * 3 * 128 * 2
        assert lib.gpt2_gen_alloc(h, 4, 64, None, 0, ctypes.byref(need), None) == 0 and need.value > n1
        g = ctypes.c_void_p()
        assert lib.gpt2_gen_alloc(h, 2, 64, ctypes.c_void_p(1 << 41), n1 - 1, None, ctypes.byref(g)) == -2
        assert lib.gpt2_gen_alloc(h, 2, 64, ctypes.c_void_p((1 << 41) + 64), n1, None, ctypes.byref(g)) == -3
        assert not g.value
        # a state over a fake address: only calls that fail validation are made with it
        assert lib.gpt2_gen_alloc(h, 2, 64, ctypes.c_void_p(1 << 41), n1, None, ctypes.byref(g)) == 0
        try:
            assert lib.gpt2_gen_length(g) == 0
            fake = ctypes.c_void_p(1 << 42)
            assert lib.gpt2_gen_decode(g, fake, fake, None) == -4        # no prefill yet
            assert lib.gpt2_gen_prefill(g, fake, 0, fake, None) == -2    # empty prompt
            assert lib.gpt2_gen_prefill(g, fake, 65, fake, None) == -2   # longer than max_len
            assert lib.gpt2_gen_prefill(g, None, 4, fake, None) == -1
        finally:
            lib.gpt2_gen_free(g)
        assert lib.gpt2_gen_length(None) == -1
    finally:
        lib.gpt2_free_arena(h)


def test_decode_noalloc_rejects_rows_beyond_its_static_array_without_touching_memory():
    # C = 1600 (head size 64): batch 16 needs about 512 KiB of decode rows, more than the
    # 384 KiB static array, and is refused before any GPU call; batch 12 fits and then
    # fails the state check (no prefill yet).
    b = _lib()
    lib = b.lib()
    m = synth.ModelShape(16, 301, 1, 25, 1600)
    cfg = b.make_config(m)
    h = ctypes.c_void_p()
    n = b.arena_bytes(m, 16, 4, b.GPT2_BF16)
    assert lib.gpt2_alloc_arena(ctypes.byref(cfg), 16, 4, 1, ctypes.c_void_p(1 << 40), n, None, ctypes.byref(h)) == 0
    try:
        fake = ctypes.c_void_p(1 << 42)
        assert lib.gpt2_gen_decode_noalloc(None, fake, fake, None) == -1
        for batch, rc in ((16, -2), (12, -4)):
            need = ctypes.c_size_t()
            assert lib.gpt2_gen_alloc(h, batch, 4, None, 0, ctypes.byref(need), None) == 0
            g = ctypes.c_void_p()
            assert lib.gpt2_gen_alloc(h, batch, 4, ctypes.c_void_p(1 << 41), need.value, None, ctypes.byref(g)) == 0
            try:
                assert lib.gpt2_gen_decode_noalloc(g, fake, fake, None) == rc, batch
                if rc == -2:
                    assert b"static scratch" in lib.gpt2_last_error()
            finally:
                lib.gpt2_gen_free(g)
    finally:
        lib.gpt2_free_arena(h)
