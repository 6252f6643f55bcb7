"""Checkpoints and token files on the GPU path: a run resumed from a checkpoint in a
fresh arena continues bit for bit where the saved run went on, with its batches read
from an int32 token file (through the C ABI)."""
import numpy as np
import pytest

import synth
from synth import ModelShape, Workload
from parity_util import FP32_LOSS_REL, gpu_arena, rand_params, to_np

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_resume_from_checkpoint_is_bitwise(dtype, tmp_path):
    from transformer_lm_fwd_amd import binding as b
    w = Workload("resume", ModelShape(160, 301, 2, 2, 128), 2, 64, dtype, "zipf", index=40)
    print(f"\n[case] resume_{dtype}: B={w.B} T={w.T}", flush=True)
    ids = synth.token_windows(w, seed=40, B=9, T=w.T).reshape(-1).astype(np.int32)  # 9 rows -> 4 batches
    path = str(tmp_path / "train.bin")
    ids.tofile(path)
    nb = b.tokens_count(path) // (w.B * w.T)
    assert nb == 4

    def batch(i):
        return b.tokens_batch(path, w.B, w.T, i % nb)

    p = rand_params(w.model, seed=40)
    a = gpu_arena(w, p)
    for t in (1, 2, 3):
        a.step(*batch(t - 1), w, t)
    ck = str(tmp_path / "ck.bin")
    a.save_checkpoint(ck, 3)
    losses = []
    for t in (4, 5, 6):
        x, y = batch(t - 1)
        a.step(x, y, w, t)
        losses.append(a.loss())
    final = to_np(a.tensor(b.T_PARAMS)).copy()
    a.close()

    r = gpu_arena(w, synth.init_params(w.model))   # different weights before the load
    t0 = r.load_checkpoint(ck)
    assert t0 == 3
    resumed = []
    for t in (4, 5, 6):
        x, y = batch(t - 1)
        r.step(x, y, w, t)
        resumed.append(r.loss())
    assert resumed == losses
    np.testing.assert_array_equal(to_np(r.tensor(b.T_PARAMS)), final)


def test_weights_only_checkpoint_reproduces_the_forward_pass(tmp_path):
    from transformer_lm_fwd_amd import binding as b
    w = Workload("wonly", ModelShape(160, 301, 2, 2, 128), 2, 64, "bf16", "uniform", index=41)
    print("\n[case] weights_only_checkpoint", flush=True)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, rand_params(w.model, seed=41))
    a.forward(x, y)
    ref = to_np(a.tensor(b.T_LOGITS)).copy()
    ck = str(tmp_path / "w.bin")
    a.save_checkpoint(ck, 0, moments=False)
    a.close()
    r = gpu_arena(w, synth.init_params(w.model))
    assert r.load_checkpoint(ck) == 0
    r.forward(x, y)
    np.testing.assert_array_equal(to_np(r.tensor(b.T_LOGITS)), ref)
    assert not to_np(r.tensor(b.T_ADAM_M)).any()   # a weights-only file leaves the moments as they were


def test_eval_loss_over_a_token_file_matches_the_oracle(tmp_path):
    import oracle
    from parity_util import oracle_model
    from transformer_lm_fwd_amd import binding as b
    w = Workload("val", ModelShape(160, 301, 2, 2, 128), 2, 64, "fp32", "zipf", index=42)
    print("\n[case] eval_loss_fp32", flush=True)
    ids = synth.token_windows(w, seed=42, B=7, T=w.T).reshape(-1).astype(np.int32)
    path = str(tmp_path / "val.bin")
    ids.tofile(path)
    p = rand_params(w.model, seed=42)
    a = gpu_arena(w, p)
    got = a.eval_loss(path, 3)
    o = oracle_model(w, p)
    ref = 0.0
    for i in range(3):
        x, y = oracle.token_batch(ids, w.B, w.T, i)
        ref += o.forward(x, y) / 3
    print(f"eval loss {got:.7f} oracle {ref:.7f}", flush=True)
    assert abs(got - ref) <= FP32_LOSS_REL * abs(ref)
    # the mean is taken behind the C ABI in batch order: averaging the per-batch
    # forward losses one by one gives it to a few fp32 ulps (a fused multiply-add may
    # round once where this sum rounds twice)
    by_one = np.float32(0.0)
    for i in range(3):
        x, y = oracle.token_batch(ids, w.B, w.T, i)
        a.forward(x, y)
        by_one = np.float32(by_one + np.float32(a.loss()) * np.float32(1 / 3))
    assert abs(got - float(by_one)) <= 4 * float(np.spacing(by_one))
    # the logits now hold a validation batch's gradient: no backward pass may follow
    a.eval_loss(path, 1)
    with pytest.raises(b.Gpt2Error):
        a.backward()
    a.close()
