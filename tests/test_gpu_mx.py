"""MX FP8 products on the GPU, through the C ABI.

* Quantization: codes and scales must equal the oracle's (oracle/mx.py) bit for bit on
  the same bf16 values - every decision (block exponent, nearest-even code) is exact
  in both.
* The block-scaled product: against the oracle's product of the dequantized
  operands (float64), to fp32 accumulation and bf16 output rounding.
* The forward pass with MX products, against the oracle's float64 forward without
  quantization: the tolerance there is the format's own error (see
  MX_LOGIT_COS and MX_LOSS_REL)."""
import numpy as np
import pytest

import oracle
import synth
from oracle import mx
from synth import ModelShape, Workload
from parity_util import cosine, gpu_arena, oracle_model, rand_params, to_np

pytestmark = pytest.mark.gpu


def announce(name, **kw):
    print(f"\n[case] {name}: " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def bf16_matrix(rows, K, seed, spread=8):
    """bf16 values whose 32-blocks span 2^-spread .. 2^spread in magnitude, with an
    all-zero block, tiny negatives (codes -0) and exact midpoints mixed in."""
    import torch
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)) * np.exp2(rng.integers(-spread, spread + 1, (rows, (K + 31) // 32))).repeat(32, 1)[:, :K]
    if K >= 64:
        x[0, 32:64] = 0.0
    x[1 % rows, :8] = -1e-30
    if K >= 16:
        x[2 % rows, 8:16] = [1.0625, 1.1875, -3.25, 448.0, 416.0 + 16, 0.0, -0.0, 2.0 ** -10]
    t = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
    return t.cuda(), t.float().numpy().astype(np.float64)


def scales_to_e(sc, K):
    """GPU scale words [Kp / 128, rows, 4] -> exponents [rows, Kp / 32]."""
    s = to_np(sc).astype(np.int64)  # [stages, rows, 4]
    return s.transpose(1, 0, 2).reshape(s.shape[1], -1) - 127


@pytest.mark.parametrize("rows,K", [(37, 768), (5, 200), (256, 3072), (1, 8), (130, 128)])
def test_quantize_matches_the_oracle_bitwise(rows, K):
    from transformer_lm_fwd_amd import binding as b
    announce("mx_quantize", rows=rows, K=K)
    x, xv = bf16_matrix(rows, K, seed=rows * 1000 + K)
    q, sc = b.mx_quantize(x)
    Kp = (K + 127) // 128 * 128
    ref_q, ref_e = mx.quantize(np.pad(xv, ((0, 0), (0, Kp - K))))
    got_q, got_e = to_np(q), scales_to_e(sc, Kp)
    np.testing.assert_array_equal(got_e, ref_e)
    np.testing.assert_array_equal(got_q, ref_q)


def _mx_case(M, N, K, seed):
    from transformer_lm_fwd_amd import binding as b
    xa, _ = bf16_matrix(M, K, seed, spread=3)
    xb, _ = bf16_matrix(N, K, seed + 1, spread=3)
    qa, sa = b.mx_quantize(xa)
    qb, sb = b.mx_quantize(xb)
    A = mx.dequantize(to_np(qa), scales_to_e(sa, K))
    Bm = mx.dequantize(to_np(qb), scales_to_e(sb, K))
    return (qa, sa, qb, sb), A, Bm


def _tol(A, Bm, ref):
    # Accumulation: a sequential fp32 sum of K terms is off by at most K 2^-24 sum |a b|.
    # The matrix core adds the 64 products of one block-scaled MFMA in its own internal
    # format (the ISA does not specify it); on these inputs its error reached 1.44 times
    # that sequential bound, so the bound is taken four times over.  Output: bf16 (2^-9
    # relative, doubled).  A wrong scale, code or lane layout is off by O(1) relative.
    K = A.shape[1]
    return 2.0 ** -8 * np.abs(ref) + 4 * K * 2.0 ** -24 * (np.abs(A) @ np.abs(Bm).T) + 1e-30


@pytest.mark.parametrize("M,N,K", [(300, 520, 384), (128, 256, 128), (8192, 768, 3072), (77, 50257, 768)])
def test_gemm_matches_the_oracle_product(M, N, K):
    import torch
    from transformer_lm_fwd_amd import binding as b
    announce("mx_gemm", M=M, N=N, K=K)
    ops, A, Bm = _mx_case(M, N, K, seed=M + N + K)
    rng = np.random.default_rng(5)
    bias = rng.standard_normal(N).astype(np.float32)
    got = to_np(b.mx_gemm(*ops, b.GPT2_EPI_BIAS, torch.tensor(bias).cuda())).astype(np.float64)
    if M * N > 4e7:  # sampled rows at the largest shapes
        rows = np.unique(np.r_[0, M - 1, rng.integers(0, M, 64)])
        A, got = A[rows], got[rows]
    ref = A @ Bm.T + bias
    err = np.abs(got - ref)
    print(f"max |C - oracle| = {err.max():.4g} (max |C| {np.abs(ref).max():.4g})", flush=True)
    assert np.all(err <= _tol(A, Bm, ref) + 2.0 ** -8 * np.abs(bias))


def test_gemm_residual_and_gelu_epilogues():
    import torch
    from transformer_lm_fwd_amd import binding as b
    M, N, K = 200, 264, 256
    announce("mx_gemm_epilogues", M=M, N=N, K=K)
    ops, A, Bm = _mx_case(M, N, K, seed=9)
    rng = np.random.default_rng(6)
    bias = torch.tensor(rng.standard_normal(N).astype(np.float32)).cuda()
    res = torch.tensor(rng.standard_normal((M, N)), dtype=torch.float32).to(torch.bfloat16).cuda()
    prod = A @ Bm.T + to_np(bias).astype(np.float64)
    got = to_np(b.mx_gemm(*ops, b.GPT2_EPI_BIAS_RES, bias, res)).astype(np.float64)
    ref = prod + to_np(res).astype(np.float64)
    assert np.all(np.abs(got - ref) <= _tol(A, Bm, ref) + 2.0 ** -8 * (np.abs(prod) + 1))
    pre, post = b.mx_gemm(*ops, b.GPT2_EPI_BIAS_GELU, bias)
    pre, post = to_np(pre).astype(np.float64), to_np(post).astype(np.float64)
    assert np.all(np.abs(pre - prod) <= _tol(A, Bm, prod) + 2.0 ** -8 * (np.abs(prod) + 1))
    # GELU of the fp32 pre-activation: tanh-GELU's slope is at most 1.13, so the
    # accumulation error passes through scaled by that; then the bf16 rounding of GELU
    g = oracle.gelu(prod)
    acc_err = _tol(A, Bm, prod) - 2.0 ** -8 * np.abs(prod)
    assert np.all(np.abs(post - g) <= 1.13 * acc_err + 2.0 ** -8 * np.abs(g) + 1e-6)


def test_gemm_rejects_bad_shapes():
    import ctypes
    from transformer_lm_fwd_amd import binding as b
    L = b.lib()
    p = ctypes.c_void_p(16)
    # K not a multiple of 128, lda < K, unknown epilogue
    for K, lda, epi in [(96, 128, 0), (128, 64, 0), (128, 128, 7)]:
        rc = L.gpt2_mx_gemm(p, p, lda, p, p, 128, p, 64, 4, 64, K, epi, None, None, None, None)
        assert rc == -1


# ---------------------------------------------------------------------------- forward pass
# Tolerance of the forward pass with MX products against the float64 oracle without
# quantization.  An E4M3 code carries 3 mantissa bits: each operand of a product is off
# by at most 2^-4 relative (RMS about 2^-4 / sqrt(3) = 0.036 for uniformly placed
# values), so a product of two quantized operands has an RMS relative error near
# 0.05 per term, which averages over the K terms of each output: one product's
# output is off by a relative RMS of about 0.05, a row cosine of 1 - 0.05^2 / 2.  The
# logits come after 4 L + 1 such products whose errors partly compound (measured:
# cosine 0.9990 for 2 layers, 0.9924 for GPT-2 124M's 12, loss within 3e-4
# relative); the bounds leave room for that growth, while a wrong scale, code or
# layout gives cosines near 0 and losses off by whole units.
MX_LOGIT_COS = 0.98
MX_LOSS_REL = 2e-2


def _forward_case(w, params, x, y):
    # logits from a forward pass without targets (with targets the fused cross-entropy
    # writes its gradient over them), the loss from one with
    from transformer_lm_fwd_amd import binding as b

    def run(a):
        a.forward(x)
        z = to_np(a.tensor(b.T_LOGITS)).astype(np.float64).copy()
        a.forward(x, y)
        return a.loss(), z

    a = gpu_arena(w, params)
    bf = run(a)
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    mxr = run(a)
    a.set_gemm_format(b.GPT2_GEMM_BF16)
    again = run(a)
    np.testing.assert_array_equal(again[1], bf[1])   # switching back restores the bf16 path bitwise
    o = oracle_model(w, params, prec="f64")
    ref_loss = o.forward(x, y)
    ref = o.act("logits").reshape(w.B * w.T, -1)
    return bf, mxr, ref_loss, ref


@pytest.mark.parametrize("name,m,B,T", [("small", ModelShape(160, 301, 2, 2, 128), 2, 64),
                                        ("gpt2_124m", synth.WORKLOADS["gpt2_124m_b8t1024_bf16"].model, 4, 64)])
def test_mx_forward_against_the_oracle(name, m, B, T):
    w = Workload(f"mx_{name}", m, B, T, "bf16", "zipf", index=50)
    announce(f"mx_forward_{name}", L=m.num_layers, C=m.channels, B=B, T=T)
    params = rand_params(m, seed=50) if name == "small" else synth.init_params(m)
    x, y = synth.inputs_targets(w)
    (bf_loss, bf_z), (mx_loss, mx_z), ref_loss, ref = _forward_case(w, params, x, y)
    V = m.vocab_size
    bf_z, mx_z = bf_z[:, :V], mx_z[:, :V]
    cos_mx = min(cosine(mx_z[r], ref[r]) for r in range(ref.shape[0]))
    cos_bf = min(cosine(bf_z[r], ref[r]) for r in range(ref.shape[0]))
    print(f"loss: oracle {ref_loss:.6f} bf16 {bf_loss:.6f} mxfp8 {mx_loss:.6f} "
          f"(rel {abs(mx_loss - ref_loss) / ref_loss:.2e}); min row cosine bf16 {cos_bf:.6f} mxfp8 {cos_mx:.6f}; "
          f"max |dz| bf16 {np.abs(bf_z - ref).max():.3g} mxfp8 {np.abs(mx_z - ref).max():.3g}", flush=True)
    assert abs(mx_loss - ref_loss) <= MX_LOSS_REL * ref_loss
    assert cos_mx >= MX_LOGIT_COS
    # the quantization must actually be on: MX logits differ from the bf16 path's
    assert np.abs(mx_z - bf_z).max() > 0


def test_mx_weights_follow_every_update():
    # after AdamW steps the MX codes must be remade: an arena that trained in MX mode
    # and a fresh arena loaded with its weights give the same MX forward, bitwise
    from transformer_lm_fwd_amd import binding as b
    w = Workload("mx_train", ModelShape(160, 301, 2, 2, 128), 2, 64, "bf16", "uniform", index=51)
    announce("mx_weights_refresh", B=w.B, T=w.T)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, rand_params(w.model, seed=51))
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    losses = []
    for t in (1, 2, 3):
        a.step(x, y, w, t)
        losses.append(a.loss())
    a.forward(x, y)
    z1 = to_np(a.tensor(b.T_LOGITS)).copy()
    p = to_np(a.tensor(b.T_PARAMS)).copy()
    r = gpu_arena(w, p)
    r.set_gemm_format(b.GPT2_GEMM_MXFP8)
    r.forward(x, y)
    np.testing.assert_array_equal(to_np(r.tensor(b.T_LOGITS)), z1)
    assert losses[-1] < losses[0]   # training through MX forward products still lowers the loss


def test_producer_written_codes_equal_the_quantizer_of_the_stored_activations():
    # In MX mode LayerNorm and the fc product's GELU epilogue write the codes of their
    # bf16 outputs themselves; they must be exactly what gpt2_mx_quantize makes of the
    # stored activations (and so, by the test above, what the oracle makes).
    from transformer_lm_fwd_amd import binding as b
    for m, B, T in [(ModelShape(160, 301, 2, 2, 128), 2, 64), (ModelShape(64, 97, 1, 3, 96), 3, 40)]:
        w = Workload("mx_fused", m, B, T, "bf16", "uniform", index=52)
        announce("mx_fused_codes", C=m.channels, B=B, T=T)
        x, y = synth.inputs_targets(w)
        a = gpu_arena(w, rand_params(m, seed=52))
        a.set_gemm_format(b.GPT2_GEMM_MXFP8)
        a.forward(x, y)
        q, sc = a.mx_buffer(b.GPT2_MX_BUF_INPUT)
        rq, rs = b.mx_quantize(a.tensor(b.T_LNF))
        np.testing.assert_array_equal(to_np(q), to_np(rq))
        np.testing.assert_array_equal(to_np(sc), to_np(rs))
        if (4 * m.channels) % 128 == 0:
            q, sc = a.mx_buffer(b.GPT2_MX_BUF_GELU)
            rq, rs = b.mx_quantize(a.tensor(b.T_FCH_GELU, m.num_layers - 1))
            np.testing.assert_array_equal(to_np(q), to_np(rq))
            np.testing.assert_array_equal(to_np(sc), to_np(rs))


def test_empty_calls_are_no_ops():
    import ctypes
    from transformer_lm_fwd_amd import binding as b
    L = b.lib()
    p = ctypes.c_void_p(16)
    assert L.gpt2_mx_quantize(p, 8, 0, 64, p, 128, p, None) == 0
    assert L.gpt2_mx_quantize(p, 8, 5, 0, p, 128, p, None) == 0
    assert L.gpt2_mx_gemm(p, p, 128, p, p, 128, p, 64, 0, 64, 128, 0, None, None, None, None) == 0
    assert L.gpt2_mx_gemm(p, p, 128, p, p, 128, p, 64, 4, 0, 128, 0, None, None, None, None) == 0


@pytest.mark.parametrize("B,T", [(1, 1), (3, 37)])
def test_mx_forward_single_position_and_ragged_rows(B, T):
    # B*T = 1 and 111 rows: one partial 128-row tile of every MX product
    m = ModelShape(64, 301, 2, 2, 128)
    w = Workload("mx_edge", m, B, T, "bf16", "uniform", index=53)
    announce("mx_forward_edge", B=B, T=T)
    params = rand_params(m, seed=53)
    x, y = synth.inputs_targets(w)
    (bf_loss, bf_z), (mx_loss, mx_z), ref_loss, ref = _forward_case(w, params, x, y)
    V = m.vocab_size
    cos = min(cosine(mx_z[r, :V], ref[r]) for r in range(ref.shape[0]))
    print(f"loss oracle {ref_loss:.6f} mxfp8 {mx_loss:.6f}; min row cosine {cos:.6f}", flush=True)
    assert abs(mx_loss - ref_loss) <= MX_LOSS_REL * ref_loss and cos >= MX_LOGIT_COS


def test_mx_forward_gpt2_350m_full_size_against_the_bf16_path():
    # GPT-2 350M at B=8, T=1024 (beyond the oracle at this size): the MX forward must keep
    # the bf16 forward's logits' direction and loss within the format's tolerance
    from transformer_lm_fwd_amd import binding as b
    w = synth.WORKLOADS["gpt2_350m_b8t1024_bf16_zipf"]
    announce("mx_forward_350m", B=w.B, T=w.T)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, synth.init_params(w.model))
    rows = np.unique(np.r_[0, w.B * w.T - 1, np.random.default_rng(1).integers(0, w.B * w.T, 62)])
    V = w.model.vocab_size

    def run():
        a.forward(x)
        z = to_np(a.tensor(b.T_LOGITS)[rows]).astype(np.float64)[:, :V]
        a.forward(x, y)
        return a.loss(), z

    lb, zb = run()
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    lm, zm = run()
    cos = min(cosine(zm[i], zb[i]) for i in range(len(rows)))
    print(f"350M loss bf16 {lb:.5f} mxfp8 {lm:.5f}; min sampled row cosine {cos:.6f}", flush=True)
    assert abs(lm - lb) <= MX_LOSS_REL * lb and cos >= MX_LOGIT_COS
