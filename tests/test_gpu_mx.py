"""MX FP8 products on the GPU, through the C ABI.

* Quantization: codes and scales must equal the oracle's (oracle/mx.py) bit for bit on
  the same bf16 values - every decision (block exponent, nearest-even code) is exact
  in both.
* The block-scaled product: against the oracle's product of the dequantized
  operands (float64), to fp32 accumulation and bf16 output rounding.
* The forward pass with MX products, against the oracle in MX mode (the same encoding
  of every product's operands, float64 products) at bf16 tolerances; the oracle without
  quantization is printed beside it (the format's own error)."""
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
# The forward pass with MX products is compared with the oracle in MX mode (each of the
# five forward products multiplies its bf16 input and weight through the same MX
# encoding, in float64): what remains is the GPU's bf16 storage of the activations, its
# fp32 accumulation, and the elements whose bf16 value differs by an ulp and so land on
# the other side of an E4M3 rounding boundary (an eighth of their value apart); such
# flips compound over the layers: measured min logit-row cosines 0.99935 (2 layers) and
# 0.9953 (GPT-2 124M, 12 layers, loss within 1e-4).  Bounds: the stated bf16 loss
# tolerance and a row cosine of 0.99.  The tight pin is layer by layer
# (test_mx_products_layer_by_layer): every product fed the GPU's own stored bf16 input,
# against the oracle's encoding and a float64 product.  The plain oracle is printed
# beside (the format's own error: cosine about 0.993 at GPT-2 124M).
MX_ORACLE_LOSS_ABS = 2e-2
MX_ORACLE_COS = 0.99
MX_PREFIX_LOSS_ABS = 5e-2


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
    o.set_mx(True)
    mx_ref_loss = o.forward(x, y)
    mx_ref = o.act("logits").reshape(w.B * w.T, -1)
    o.close()
    return bf, mxr, (ref_loss, ref), (mx_ref_loss, mx_ref)


def _row_cos(z, ref):
    return min(cosine(z[r], ref[r]) for r in range(ref.shape[0]))


@pytest.mark.parametrize("name,m,B,T", [("small", ModelShape(160, 301, 2, 2, 128), 2, 64),
                                        ("gpt2_124m", synth.WORKLOADS["gpt2_124m_b8t1024_bf16"].model, 4, 64)])
def test_mx_forward_against_the_oracle(name, m, B, T):
    w = Workload(f"mx_{name}", m, B, T, "bf16", "zipf", index=50)
    announce(f"mx_forward_{name}", L=m.num_layers, C=m.channels, B=B, T=T)
    params = rand_params(m, seed=50) if name == "small" else synth.init_params(m)
    x, y = synth.inputs_targets(w)
    (bf_loss, bf_z), (mx_loss, mx_z), (ref_loss, ref), (mref_loss, mref) = _forward_case(w, params, x, y)
    V = m.vocab_size
    bf_z, mx_z = bf_z[:, :V], mx_z[:, :V]
    cos_mx, cos_plain, cos_bf = _row_cos(mx_z, mref), _row_cos(mx_z, ref), _row_cos(bf_z, ref)
    mean_mx = float(np.mean([cosine(mx_z[r], mref[r]) for r in range(mref.shape[0])]))
    print(f"mean row cosine MX vs MX oracle {mean_mx:.6f}", flush=True)
    print(f"loss: MX oracle {mref_loss:.6f} GPU MX {mx_loss:.6f} (|d| {abs(mx_loss - mref_loss):.2e}); "
          f"oracle {ref_loss:.6f} GPU bf16 {bf_loss:.6f}; min row cosine: MX vs MX oracle {cos_mx:.6f}, "
          f"MX vs plain oracle {cos_plain:.6f}, bf16 vs plain oracle {cos_bf:.6f}", flush=True)
    assert abs(mx_loss - mref_loss) <= MX_ORACLE_LOSS_ABS
    assert cos_mx >= MX_ORACLE_COS
    # the quantization must actually be on: MX logits differ from the bf16 path's
    assert np.abs(mx_z - bf_z).max() > 0


def test_mx_training_gradients_against_the_oracle():
    # A training step with MX forward products: the backward pass takes the stored bf16
    # activations and weights as they are (straight-through), on both sides.
    from transformer_lm_fwd_amd import binding as b
    m = ModelShape(160, 301, 2, 2, 128)
    w = Workload("mx_grad", m, 2, 64, "bf16", "uniform", index=54)
    announce("mx_training_gradients", L=m.num_layers, C=m.channels, B=w.B, T=w.T)
    params = rand_params(m, seed=54)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, params)
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    a.forward(x, y)
    loss = a.loss()
    a.backward()
    g = to_np(a.tensor(b.T_GRADS)).ravel()
    a.close()
    o = oracle_model(w, params, prec="f64")
    o.set_mx(True)
    ref = o.forward(x, y)
    o.backward()
    gr = o.get("grads")
    o.close()
    cos = cosine(g, gr)
    print(f"MX step: loss GPU {loss:.6f} MX oracle {ref:.6f}; flat gradient cosine {cos:.6f}", flush=True)
    assert abs(loss - ref) <= MX_ORACLE_LOSS_ABS
    assert cos >= 0.999


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
    # In MX mode LayerNorm, the fc product's GELU epilogue and (MX dX format) the
    # softmax-CE write the codes of their bf16 outputs themselves; they must be exactly
    # what gpt2_mx_quantize makes of the stored tensors (and so, by the test above, what
    # the oracle makes).
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
        # under GPT2_GEMM_MXFP8_DX the softmax-CE kernel writes the codes of the logits'
        # gradient: from registers for the 128-value stages inside the full vectors of a
        # row, by reading the row back for the rest (V = 301: stages 0-1, then stage 2)
        a.set_gemm_format(b.GPT2_GEMM_MXFP8_DX)
        a.forward(x, y)
        q, sc = a.mx_buffer(b.GPT2_MX_BUF_DY)
        z = a.tensor(b.T_LOGITS)  # [B*T, V] view of rows of the padded width (the CE writes the padding as 0)
        rq, rs = b.mx_quantize(z.as_strided((z.shape[0], z.stride(0)), (z.stride(0), 1)))
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


def _mx_op(x):
    """The operand an MX product multiplies (oracle/mx.py's encoder): the bf16 values x
    [rows, K], zero-padded to whole 32-blocks, encoded and decoded."""
    R, K = x.shape
    Kp = (K + 31) // 32 * 32
    return mx.dequantize(*mx.quantize(np.pad(x, ((0, 0), (0, Kp - K)))))[:, :K]


def _bf16_np(x):
    import torch
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("name,m,B,T", [("small", ModelShape(160, 301, 2, 2, 128), 2, 64),
                                        ("gpt2_124m", synth.WORKLOADS["gpt2_124m_b8t1024_bf16"].model, 4, 64),
                                        ("gpt2_350m", synth.WORKLOADS["gpt2_350m_b8t1024_bf16_zipf"].model, 2, 32)])
def test_mx_products_layer_by_layer(name, m, B, T):
    # Every MX product of the forward pass, fed the GPU's own stored bf16 input (so no
    # upstream difference can flip a code): qkv, the attention projection with its
    # residual, c_fc with GELU, the c_fc projection with its residual, the tied lm_head.
    # Reference: oracle/mx.py's encoding of input and bf16 weight, float64 product, the
    # bias and residual added in float64; tolerance: fp32 accumulation (as in the GEMM
    # test) plus the bf16 rounding of the stored output.
    from transformer_lm_fwd_amd import binding as b
    w = Workload(f"mx_ltl_{name}", m, B, T, "bf16", "uniform", index=55)
    announce(f"mx_products_layer_by_layer_{name}", L=m.num_layers, C=m.channels, B=B, T=T)
    params = rand_params(m, seed=55) if name == "small" else synth.init_params(m)
    x, _ = synth.inputs_targets(w)
    a = gpu_arena(w, params)
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    a.forward(x)
    offs = synth.param_offsets(m)

    def act(tid, l=0):
        return to_np(a.tensor(tid, l)).astype(np.float64)

    def P(name):
        o, n = offs[name]
        return np.asarray(params[o:o + n], dtype=np.float64)

    worst = 0.0

    def check(label, out, inp, wname, bias=None, resid=None, gelu_out=None):
        nonlocal worst
        Wm = _bf16_np(P(wname).reshape(-1, inp.shape[1]))
        A, Bm = _mx_op(inp), _mx_op(Wm)
        prod = A @ Bm.T
        if bias is not None:
            prod = prod + bias
        acc_err = 4 * inp.shape[1] * 2.0 ** -24 * (np.abs(A) @ np.abs(Bm).T)
        ref = prod if resid is None else prod + resid
        err = np.abs(out - ref)
        tol = 2.0 ** -8 * np.abs(ref) + acc_err + 1e-30
        worst = max(worst, float((err / tol).max()))
        assert np.all(err <= tol), (label, float((err / tol).max()))
        if gelu_out is not None:
            g = oracle.gelu(prod)
            assert np.all(np.abs(gelu_out - g) <= 1.13 * acc_err + 2.0 ** -8 * np.abs(g) + 1e-6), label + " gelu"

    for l in range(m.num_layers):
        h = f"h{l}."
        xin = act(b.T_ENCODED) if l == 0 else act(b.T_RESIDUAL3, l - 1)
        check(f"qkv{l}", act(b.T_QKV, l), act(b.T_LN1, l), h + "qkv.w", P(h + "qkv.b"))
        check(f"proj{l}", act(b.T_RESIDUAL2, l), act(b.T_ATTY, l), h + "proj.w", P(h + "proj.b"), resid=xin)
        check(f"fc{l}", act(b.T_FCH, l), act(b.T_LN2, l), h + "fc.w", P(h + "fc.b"), gelu_out=act(b.T_FCH_GELU, l))
        check(f"fcproj{l}", act(b.T_RESIDUAL3, l), act(b.T_FCH_GELU, l), h + "fcproj.w", P(h + "fcproj.b"),
              resid=act(b.T_RESIDUAL2, l))
    check("lm_head", act(b.T_LOGITS), act(b.T_LNF), "wte")
    a.close()
    print(f"{4 * m.num_layers + 1} MX products within bounds (largest error / bound {worst:.3f})", flush=True)


def test_attention_written_codes_give_the_projection_bit_for_bit():
    # With MX products the attention kernel writes the codes of its output (head size
    # 64, C % 128 == 0) instead of a separate quantizer pass.  The attention projection
    # recomputed with gpt2_mx_quantize's codes of the stored output (same weight codes,
    # bias and residual, same kernel) must give the arena's result bit for bit.
    import torch
    from transformer_lm_fwd_amd import binding as b
    for name, m, B, T in [("small", ModelShape(160, 301, 2, 2, 128), 2, 64),
                          ("gpt2_124m", synth.WORKLOADS["gpt2_124m_b8t1024_bf16"].model, 2, 128)]:
        w = Workload(f"mx_attcodes_{name}", m, B, T, "bf16", "uniform", index=57)
        announce(f"mx_attention_codes_{name}", C=m.channels, NH=m.num_heads, B=B, T=T)
        params = rand_params(m, seed=57) if name == "small" else synth.init_params(m)
        x, _ = synth.inputs_targets(w)
        a = gpu_arena(w, params)
        a.set_gemm_format(b.GPT2_GEMM_MXFP8)
        a.forward(x)
        offs = synth.param_offsets(m)
        for l in range(m.num_layers):
            o, n = offs[f"h{l}.proj.b"]
            bias = torch.tensor(np.asarray(params[o:o + n], dtype=np.float32)).cuda()
            xin = a.tensor(b.T_ENCODED) if l == 0 else a.tensor(b.T_RESIDUAL3, l - 1)
            qa, sa = b.mx_quantize(a.tensor(b.T_ATTY, l))
            qb, sb = a.mx_weight_codes(4 * l + 1)
            got = b.mx_gemm(qa, sa, qb, sb, b.GPT2_EPI_BIAS_RES, bias, xin)
            np.testing.assert_array_equal(to_np(got), to_np(a.tensor(b.T_RESIDUAL2, l)))
        a.close()


@pytest.mark.parametrize("B,T", [(1, 1), (3, 37)])
def test_mx_forward_single_position_and_ragged_rows(B, T):
    # B*T = 1 and 111 rows: one partial 128-row tile of every MX product
    m = ModelShape(64, 301, 2, 2, 128)
    w = Workload("mx_edge", m, B, T, "bf16", "uniform", index=53)
    announce("mx_forward_edge", B=B, T=T)
    params = rand_params(m, seed=53)
    x, y = synth.inputs_targets(w)
    _, (mx_loss, mx_z), _, (mref_loss, mref) = _forward_case(w, params, x, y)
    V = m.vocab_size
    cos = _row_cos(mx_z[:, :V], mref)
    print(f"loss MX oracle {mref_loss:.6f} GPU MX {mx_loss:.6f}; min row cosine {cos:.6f}", flush=True)
    assert abs(mx_loss - mref_loss) <= MX_ORACLE_LOSS_ABS and cos >= MX_ORACLE_COS


def test_mx_forward_gpt2_350m_full_size_sampled_prefixes():
    # GPT-2 350M at B=8, T=1024 with MX products: by causality, positions 0..63 of a
    # sequence depend only on its first 64 tokens, so the oracle in MX mode on those
    # prefixes gives their logits and losses exactly.
    from transformer_lm_fwd_amd import binding as b
    w = synth.WORKLOADS["gpt2_350m_b8t1024_bf16_zipf"]
    announce("mx_forward_350m", B=w.B, T=w.T)
    params = synth.init_params(w.model)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, params)
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    V, t0 = w.model.vocab_size, 64
    a.forward(x)
    z = to_np(a.tensor(b.T_LOGITS)).astype(np.float64).reshape(w.B, w.T, -1)
    a.forward(x, y)
    losses = to_np(a.tensor(b.T_LOSSES)).reshape(w.B, w.T)
    a.close()
    for row in (0, w.B - 1):
        o = oracle_model(w, params, B=1, T=t0)
        o.set_mx(True)
        o.forward(x[row:row + 1, :t0], y[row:row + 1, :t0])
        ref_z = o.act("logits").reshape(t0, -1)
        ref_l = o.act("losses")
        o.close()
        cos = _row_cos(z[row, :t0, :V], ref_z)
        dm = abs(float(np.mean(losses[row, :t0])) - float(np.mean(ref_l)))
        print(f"row {row}: positions < {t0}: |mean loss - MX oracle| = {dm:.3g}, min row cosine {cos:.6f}",
              flush=True)
        # a mean over 64 positions of one sequence after 24 layers of E4M3 code flips
        # (measured up to 0.022); the products themselves are pinned layer by layer
        assert dm <= MX_PREFIX_LOSS_ABS and cos >= MX_ORACLE_COS


def test_gemm_gelu_backward_epilogue():
    # GPT2_EPI_GELU_BWD: C = (A B^T) * GELU'(pre), the GELU input's gradient.  GELU' is
    # at most 1.13 in magnitude, so the product's accumulation error passes through
    # scaled by that, then the bf16 rounding of C.
    import torch
    from transformer_lm_fwd_amd import binding as b
    M, N, K = 200, 264, 256
    announce("mx_gemm_gelu_bwd", M=M, N=N, K=K)
    ops, A, Bm = _mx_case(M, N, K, seed=19)
    rng = np.random.default_rng(16)
    pre = torch.tensor(rng.standard_normal((M, N)) * 2, dtype=torch.float32).to(torch.bfloat16).cuda()
    prod = A @ Bm.T
    got = to_np(b.mx_gemm(*ops, b.GPT2_EPI_GELU_BWD, None, pre)).astype(np.float64)
    gg = oracle.gelu_grad(to_np(pre).astype(np.float64))
    ref = prod * gg
    acc_err = _tol(A, Bm, prod) - 2.0 ** -8 * np.abs(prod)
    assert np.all(np.abs(got - ref) <= 1.13 * acc_err + 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_gemm_gelu_epilogues_with_64_code_k_tiles():
    # At 384 or more output tiles the two GELU epilogues run with 64-code k-tiles (two
    # blocks per CU): 4096 x 3072 x 768 has exactly 384.  Sampled rows against the oracle's
    # product, with the tolerances of the small-shape epilogue tests above.
    import torch
    from transformer_lm_fwd_amd import binding as b
    M, N, K = 4096, 3072, 768
    announce("mx_gemm_gelu_64code_tiles", M=M, N=N, K=K)
    ops, A, Bm = _mx_case(M, N, K, seed=23)
    rng = np.random.default_rng(24)
    rows = np.unique(np.r_[0, 1, M - 1, rng.integers(0, M, 48)])
    bias = torch.tensor(rng.standard_normal(N).astype(np.float32)).cuda()
    prod = A[rows] @ Bm.T
    tol = _tol(A[rows], Bm, prod)
    pre, post = b.mx_gemm(*ops, b.GPT2_EPI_BIAS_GELU, bias)
    pre, post = to_np(pre).astype(np.float64)[rows], to_np(post).astype(np.float64)[rows]
    pb = prod + to_np(bias).astype(np.float64)
    assert np.all(np.abs(pre - pb) <= _tol(A[rows], Bm, pb) + 2.0 ** -8)
    g = oracle.gelu(pb)
    acc_err = tol - 2.0 ** -8 * np.abs(prod)
    assert np.all(np.abs(post - g) <= 1.13 * acc_err + 2.0 ** -8 * np.abs(g) + 1e-6)
    x = torch.tensor(rng.standard_normal((M, N)) * 2, dtype=torch.float32).to(torch.bfloat16).cuda()
    got = to_np(b.mx_gemm(*ops, b.GPT2_EPI_GELU_BWD, None, x)).astype(np.float64)[rows]
    ref = prod * oracle.gelu_grad(to_np(x).astype(np.float64)[rows])
    assert np.all(np.abs(got - ref) <= 1.13 * acc_err + 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_mx_dx_transposed_weight_codes_equal_the_quantizer_of_the_transposes():
    # Under GPT2_GEMM_MXFP8_DX the forward pass's code refresh also makes the codes of
    # every weight's transpose (blocks of 32 along the layer's outputs): they must equal
    # the quantizer run on the transposed bf16 weights, bit for bit, with the columns
    # past the outputs (the vocabulary's padding for the tied embedding) as zero.
    import torch
    from transformer_lm_fwd_amd import binding as b
    m = ModelShape(160, 301, 2, 2, 128)
    w = Workload("mx_dx_codes", m, 2, 64, "bf16", "uniform", index=62)
    announce("mx_dx_weight_codes", L=m.num_layers, C=m.channels, V=m.vocab_size)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, rand_params(m, seed=62))
    a.set_gemm_format(b.GPT2_GEMM_MXFP8_DX)
    a.forward(x, y)
    torch.cuda.synchronize()
    p16 = a.tensor(b.T_PARAMS_BF16).view(-1)
    offs = synth.param_offsets(m)
    C = m.channels
    names = [("h0.qkv.w", 3 * C, C), ("h0.proj.w", C, C), ("h1.fc.w", 4 * C, C), ("h1.fcproj.w", C, 4 * C),
             ("wte", m.vocab_size, C)]
    idx = [0, 1, 6, 7, 4 * m.num_layers]
    for (name, rows, k), i in zip(names, idx):
        off, n = offs[name]
        W = p16[off:off + n].view(rows, k)
        rp = (rows + 127) // 128 * 128
        wt = torch.zeros(k, rp, dtype=torch.bfloat16, device=W.device)
        wt[:, :rows] = W.t()
        q_ref, s_ref = b.mx_quantize(wt)
        q, s = a.mx_weight_codes(i, transposed=True)
        assert tuple(q.shape) == (k, rp)
        assert torch.equal(q, q_ref[:, :rp]), name
        assert torch.equal(s, s_ref), name
        # and the forward codes are those of W itself
        qf, sf = a.mx_weight_codes(i, transposed=False)
        q_f, s_f = b.mx_quantize(W.contiguous())
        assert torch.equal(qf, q_f[:, :qf.shape[1]]) and torch.equal(sf, s_f), name
    a.close()


def test_mx_dx_training_gradients_against_the_oracle():
    # GPT2_GEMM_MXFP8_DX: MX forward products and MX input-gradient products on both
    # sides (the oracle's MX mode 2); weight gradients from the plain operands.
    from transformer_lm_fwd_amd import binding as b
    m = ModelShape(160, 301, 2, 2, 128)
    w = Workload("mx_dx_grad", m, 2, 64, "bf16", "uniform", index=63)
    announce("mx_dx_training_gradients", L=m.num_layers, C=m.channels, B=w.B, T=w.T)
    params = rand_params(m, seed=63)
    x, y = synth.inputs_targets(w)
    a = gpu_arena(w, params)
    a.set_gemm_format(b.GPT2_GEMM_MXFP8)
    a.forward(x, y)
    loss1 = a.loss()
    a.backward()
    g1 = to_np(a.tensor(b.T_GRADS)).ravel().copy()
    a.set_gemm_format(b.GPT2_GEMM_MXFP8_DX)
    a.forward(x, y)
    loss = a.loss()
    a.backward()
    g = to_np(a.tensor(b.T_GRADS)).ravel().copy()
    a.close()
    assert loss == loss1              # the forward pass does not depend on the dX format
    o = oracle_model(w, params, prec="f64")
    o.set_mx(2)
    ref = o.forward(x, y)
    o.backward()
    gr = o.get("grads")
    o.set_mx(1)
    o.forward(x, y)
    o.backward()
    gr1 = o.get("grads")
    o.close()
    cos, cos1 = cosine(g, gr), cosine(g, gr1)
    print(f"MX dX step: loss GPU {loss:.6f} MX oracle {ref:.6f}; flat gradient cosine {cos:.6f} "
          f"(against the oracle without MX input gradients: {cos1:.6f}; GPU modes 1 vs 2: {cosine(g, g1):.6f})",
          flush=True)
    assert abs(loss - ref) <= MX_ORACLE_LOSS_ABS
    assert cos >= 0.999
    assert not np.array_equal(g, g1)


def test_mx_dx_step_trains_and_switching_back_restores_bf16():
    from transformer_lm_fwd_amd import binding as b
    w = Workload("mx_dx_train", ModelShape(160, 301, 2, 2, 128), 2, 64, "bf16", "uniform", index=64)
    announce("mx_dx_train", B=w.B, T=w.T)
    x, y = synth.inputs_targets(w)
    p = rand_params(w.model, seed=64)
    r = gpu_arena(w, p)
    r.forward(x, y)
    r.backward()
    g_bf16 = to_np(r.tensor(b.T_GRADS)).copy()
    r.close()
    a = gpu_arena(w, p)
    a.set_gemm_format(b.GPT2_GEMM_MXFP8_DX)
    losses = []
    for t in (1, 2, 3):
        a.step(x, y, w, t)
        losses.append(a.loss())
    assert losses[-1] < losses[0]
    a.load_params(p)
    a.set_gemm_format(b.GPT2_GEMM_BF16)
    a.forward(x, y)
    a.backward()
    np.testing.assert_array_equal(to_np(a.tensor(b.T_GRADS)), g_bf16)
    a.close()
