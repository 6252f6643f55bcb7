"""Token streams, layer orders of weight files and checkpoints (host functions of the
library, through the C ABI; no GPU).  The oracle's definitions are pinned to what the
pages print, and the library is compared with them."""
import os

import numpy as np
import pytest

import oracle
import synth


def _b():
    from transformer_lm_fwd_amd import binding
    return binding


def test_oracle_batch_counts_match_the_printed_run_banner(tmp_path):
    # the llm.c run banner: 305260 training ids -> 1192 batches, 32768 validation ids ->
    # 128 batches; both fit B*T = 256 only as n // (B*T)
    for n, nb in [(305260, 1192), (32768, 128)]:
        ids = np.arange(n, dtype=np.int32)
        oracle.token_batch(ids, 4, 64, nb - 1)
        with pytest.raises(IndexError):
            oracle.token_batch(ids, 4, 64, nb)
    x, y = oracle.token_batch(np.arange(10), 1, 5, 1)   # the last batch wraps to id 0
    assert x.tolist() == [[5, 6, 7, 8, 9]] and y.tolist() == [[6, 7, 8, 9, 0]]


def test_library_token_batches_match_the_oracle(tmp_path):
    b = _b()
    rng = np.random.default_rng(3)
    for n, B, T in [(32768, 4, 64), (1001, 3, 7), (64, 2, 32)]:
        ids = rng.integers(0, 50257, n).astype(np.int32)
        path = str(tmp_path / f"tok_{n}.bin")
        ids.tofile(path)
        assert b.tokens_count(path) == n
        nb = n // (B * T)
        for i in sorted({0, 1, nb // 2, nb - 1} & set(range(nb))):
            x, y = b.tokens_batch(path, B, T, i)
            rx, ry = oracle.token_batch(ids, B, T, i)
            np.testing.assert_array_equal(x, rx)
            np.testing.assert_array_equal(y, ry)
        with pytest.raises(b.Gpt2Error):
            b.tokens_batch(path, B, T, nb)
    bad = str(tmp_path / "bad.bin")
    open(bad, "wb").write(b"\x00" * 7)
    with pytest.raises(b.Gpt2Error):
        b.tokens_count(bad)


def test_lexicographic_layer_order_pin():
    # the page: layer 0, then 1, then 10
    assert oracle.lexicographic_layer_order(12)[:3] == [0, 1, 10]
    assert oracle.lexicographic_layer_order(12) == [0, 1, 10, 11, 2, 3, 4, 5, 6, 7, 8, 9]
    assert oracle.lexicographic_layer_order(3) == [0, 1, 2]


def test_library_permutation_matches_the_oracle():
    b = _b()
    m = synth.ModelShape(64, 101, 12, 2, 32)   # 12 layers: the order differs from numeric
    n = b.num_parameters(m)
    p = np.random.default_rng(1).standard_normal(n).astype(np.float32)
    lex = b.params_permute(m, p, b.GPT2_ORDER_NUMERIC, b.GPT2_ORDER_LEXICOGRAPHIC)
    np.testing.assert_array_equal(lex, oracle.permute_layers(m, p, True))
    back = b.params_permute(m, lex, b.GPT2_ORDER_LEXICOGRAPHIC, b.GPT2_ORDER_NUMERIC)
    np.testing.assert_array_equal(back, p)
    np.testing.assert_array_equal(oracle.permute_layers(m, lex, False), p)
    # the layer blocks moved, the embeddings and ln_f did not
    head = (m.vocab_size + m.max_seq_len) * m.channels
    block = 12 * m.channels ** 2 + 13 * m.channels
    np.testing.assert_array_equal(lex[:head], p[:head])
    np.testing.assert_array_equal(lex[head + 2 * block: head + 3 * block], p[head + 10 * block: head + 11 * block])


def test_checkpoint_round_trip_and_rejections(tmp_path):
    import ctypes
    b = _b()
    m = synth.GPT2_TINY_CHAR
    n = b.num_parameters(m)
    rng = np.random.default_rng(2)
    p, mm, vv = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
    cfg = b.make_config(m)
    path = str(tmp_path / "ck.bin")
    L = b.lib()
    assert L.gpt2_checkpoint_write(path.encode(), ctypes.byref(cfg), 7, p.ctypes.data, mm.ctypes.data,
                                   vv.ctypes.data) == 0
    assert os.path.getsize(path) == 64 + 3 * 4 * n and not os.path.exists(path + ".tmp")
    q, qm, qv = (np.zeros(n, np.float32) for _ in range(3))
    step, has = ctypes.c_int32(0), ctypes.c_int32(0)
    assert L.gpt2_checkpoint_read(path.encode(), ctypes.byref(cfg), ctypes.byref(step), q.ctypes.data,
                                  qm.ctypes.data, qv.ctypes.data, ctypes.byref(has)) == 0
    assert step.value == 7 and has.value == 1
    np.testing.assert_array_equal(q, p)
    np.testing.assert_array_equal(qm, mm)
    np.testing.assert_array_equal(qv, vv)
    hdr = np.fromfile(path, dtype=np.int32, count=16)
    assert hdr[:9].tolist() == [0x32545047, 1, m.max_seq_len, m.vocab_size, m.num_layers, m.num_heads,
                                m.channels, 1, 7]
    # weights only
    path2 = str(tmp_path / "w.bin")
    assert L.gpt2_checkpoint_write(path2.encode(), ctypes.byref(cfg), 0, p.ctypes.data, None, None) == 0
    assert L.gpt2_checkpoint_read(path2.encode(), ctypes.byref(cfg), None, q.ctypes.data, qm.ctypes.data,
                                  qv.ctypes.data, ctypes.byref(has)) == 0 and has.value == 0
    # a different shape, a truncated file, a foreign file, half the moments
    other = b.make_config(synth.ModelShape(m.max_seq_len, m.vocab_size, m.num_layers, m.num_heads, m.channels * 2))
    assert L.gpt2_checkpoint_read(path.encode(), ctypes.byref(other), None, q.ctypes.data, None, None, None) == -1
    open(str(tmp_path / "short.bin"), "wb").write(open(path, "rb").read()[:1000])
    assert L.gpt2_checkpoint_read(str(tmp_path / "short.bin").encode(), ctypes.byref(cfg), None, q.ctypes.data,
                                  None, None, None) == -2
    open(str(tmp_path / "foreign.bin"), "wb").write(b"\x01" * 4096)
    assert L.gpt2_checkpoint_read(str(tmp_path / "foreign.bin").encode(), ctypes.byref(cfg), None, q.ctypes.data,
                                  None, None, None) == -1
    assert L.gpt2_checkpoint_write(path.encode(), ctypes.byref(cfg), 0, p.ctypes.data, mm.ctypes.data, None) == -1
