// GPT-2 training-step ORACLE -- test infrastructure only.
//
// A plain, slow, obviously correct CPU implementation of one GPT-2 training
// step (forward, backward, AdamW).  Only the tests, the package's smoke check
// and the CPU-baseline leg of the benchmark may load it; the GPU library never
// links, includes or calls anything here, and this file includes nothing of
// the GPU library.  It is templated on the real type: `double` is the parity
// reference, `float` is the fp32 CPU baseline (the llm.c page describes a
// CPU/fp32 trainer).
//
// Sources (cited by page title and section):
//  [llm.c]   "1000 行 C 代码完成 GPT-2 训练的 LLM.c" (bigegpt.com post 1835):
//            one up-front allocation, the layer list (encoder, layernorm, matmul,
//            self-attention, gelu, residual, softmax, cross-entropy), forward /
//            backward / Adam update loop; "快速开始吧！" run banner
//            (num_parameters 124439808, num_activations 73323776).
//  [torch-R] "GPT-2 from scratch with torch" (Posit AI Blog, Chinese translation):
//            sections 总体架构, Transformer block, 自注意力, 前馈网络（MLP）,
//            token/position embedding, 输出.
//  [c3000]   "GPT-2ベースの3000バイトCで実装されたChatGPTクローン" (hada.io):
//            sections ニューラルネットワーク層の実装, Transformer本体, and the
//            GELU formula in the comment thread.
//  [nanogpt] "从头搭建GPT(Andrej Karpathy) 笔记" (CSDN): sections 计算loss,
//            直觉上的self-attention, attention中为什么要做scaling.
//
// Readings where the pages leave a step open (all documented in the design notes):
//  * LayerNorm: biased variance over the C channels, eps = 1e-5 inside the sqrt.
//  * GELU: tanh form with sqrt(2/pi) (the comment prints its truncation .7978845).
//  * lm_head tied to wte, no bias (needed for the printed parameter count).
//  * positions 0..T-1; q|k|v column blocks, head j = columns j*hs..(j+1)*hs-1.
//  * loss = mean over all B*T positions of logsumexp(z) - z[target].
//  * no dropout; each backward overwrites the gradients.
//  * AdamW with bias correction, eps outside the sqrt, decoupled decay lr*wd*theta.
//
// Parallelism: OpenMP only over independent outputs; each output's summation
// order is fixed, so results do not depend on the thread count.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <new>
#include <string>
#include <type_traits>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

struct Shape {
    int V, P, L, NH, C;  // vocab_size, max_seq_len, num_layers, num_heads, channels
    int block = 0;       // 0: GPT-2 block; 1: Llama-style block (see llama_hidden)
};

// Llama-style block ([llm.c]: the layers to add for Llama-2-type models; [torch-R]
// names RoPE): x = x + attn(rms_1(x)), x = x + swiglu_mlp(rms_2(x)), no biases, the
// rotary position embedding instead of wpe.  RMSNorm: y = x / sqrt(mean(x^2) + eps) * w.
// SwiGLU MLP of width H: down( silu(x W_gate^T) * (x W_up^T) ), silu(g) = g sigmoid(g);
// the gate and up weights are stored interleaved, row 2j = gate_j, row 2j + 1 = up_j, so
// the product's output holds (g_j, u_j) in columns 2j, 2j + 1.  H = 8C/3 rounded up to
// a multiple of 64 (about the parameter count of a 4C GELU MLP).  The final norm is an
// RMSNorm; the lm_head stays tied to wte; wpe stays in the array, unused.
static int64_t llama_hidden(int64_t C) { return 64 * ((C + 23) / 24); }

// ----------------------------------------------------------------------------- parameter list
// Layer-major order following the module tree of [torch-R] 总体架构 / Transformer block:
// wte, wpe, then per block (ln_1, c_attn, c_proj, ln_2, c_fc, mlp c_proj), then ln_f.
enum PIdx { LN1W, LN1B, QKVW, QKVB, PROJW, PROJB, LN2W, LN2B, FCW, FCB, FCPW, FCPB, NPL };

static void layer_param_sizes(const Shape& s, int64_t out[NPL]) {
    int64_t C = s.C;
    if (s.block == 1) {  // no biases, RMSNorm gains only, gate|up and down
        const int64_t H = llama_hidden(C);
        for (int i = 0; i < NPL; ++i) out[i] = 0;
        out[LN1W] = C; out[QKVW] = 3 * C * C; out[PROJW] = C * C; out[LN2W] = C;
        out[FCW] = 2 * H * C; out[FCPW] = C * H;
        return;
    }
    out[LN1W] = C;         out[LN1B] = C;
    out[QKVW] = 3 * C * C; out[QKVB] = 3 * C;
    out[PROJW] = C * C;    out[PROJB] = C;
    out[LN2W] = C;         out[LN2B] = C;
    out[FCW] = 4 * C * C;  out[FCB] = 4 * C;
    out[FCPW] = 4 * C * C; out[FCPB] = C;
}

static int64_t count_params(const Shape& s) {
    int64_t per[NPL];
    layer_param_sizes(s, per);
    int64_t n = (int64_t)s.V * s.C + (int64_t)s.P * s.C;
    for (int l = 0; l < s.L; ++l)
        for (int i = 0; i < NPL; ++i) n += per[i];
    return n + (s.block == 1 ? 1 : 2) * (int64_t)s.C;  // final norm: w (and b for LayerNorm)
}

template <class R>
struct Params {
    R* wte;
    R* wpe;
    std::vector<R*> t[NPL];  // t[kind][layer]
    R* lnfw;
    R* lnfb;
    void bind(R* base, const Shape& s) {
        int64_t per[NPL];
        layer_param_sizes(s, per);
        R* p = base;
        wte = p; p += (int64_t)s.V * s.C;
        wpe = p; p += (int64_t)s.P * s.C;
        for (int i = 0; i < NPL; ++i) t[i].assign(s.L, nullptr);
        for (int l = 0; l < s.L; ++l)
            for (int i = 0; i < NPL; ++i) { t[i][l] = p; p += per[i]; }
        lnfw = p; p += s.C;
        lnfb = p; p += s.block == 1 ? 0 : s.C;
    }
};

// ----------------------------------------------------------------------------- activation list
// The plain activation set of the llm.c trainer: everything each layer's
// backward needs, unfused, including both B*NH*T*T attention maps.
enum AIdx {
    A_ENCODED,
    A_LN1, A_LN1_MEAN, A_LN1_RSTD, A_QKV, A_ATTY, A_PREATT, A_ATT, A_ATTPROJ, A_RESIDUAL2,
    A_LN2, A_LN2_MEAN, A_LN2_RSTD, A_FCH, A_FCH_GELU, A_FCPROJ, A_RESIDUAL3,
    A_LNF, A_LNF_MEAN, A_LNF_RSTD, A_LOGITS, A_PROBS, A_LOSSES, NACT
};
static const char* kActNames[NACT] = {
    "encoded",
    "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "preatt", "att", "attproj", "residual2",
    "ln2", "ln2_mean", "ln2_rstd", "fch", "fch_gelu", "fcproj", "residual3",
    "lnf", "lnf_mean", "lnf_rstd", "logits", "probs", "losses"};
static bool act_per_layer(int a) { return a >= A_LN1 && a <= A_RESIDUAL3; }

static int64_t act_size(const Shape& s, int B, int T, int a) {
    int64_t BT = (int64_t)B * T, C = s.C;
    switch (a) {
        case A_ENCODED: case A_LN1: case A_ATTY: case A_ATTPROJ: case A_RESIDUAL2:
        case A_LN2: case A_FCPROJ: case A_RESIDUAL3: case A_LNF:
            return BT * C;
        case A_LN1_MEAN: case A_LN1_RSTD: case A_LN2_MEAN: case A_LN2_RSTD:
        case A_LNF_MEAN: case A_LNF_RSTD: case A_LOSSES:
            return BT;
        case A_QKV: return 3 * BT * C;
        case A_PREATT: case A_ATT: return (int64_t)B * s.NH * T * T;
        case A_FCH: return s.block == 1 ? 2 * BT * llama_hidden(C) : 4 * BT * C;
        case A_FCH_GELU: return s.block == 1 ? BT * llama_hidden(C) : 4 * BT * C;
        case A_LOGITS: case A_PROBS: return BT * s.V;
    }
    return 0;
}

static int64_t count_acts(const Shape& s, int B, int T) {
    int64_t n = 0;
    for (int a = 0; a < NACT; ++a) n += act_size(s, B, T, a) * (act_per_layer(a) ? s.L : 1);
    return n;
}

template <class R>
struct Acts {
    std::vector<R> mem;
    std::vector<R*> p[NACT];  // p[a][layer] (single entry for model-level tensors)
    void alloc(const Shape& s, int B, int T) {
        mem.assign((size_t)count_acts(s, B, T), R(0));
        R* q = mem.data();
        for (int a = 0; a < NACT; ++a) {
            int n = act_per_layer(a) ? s.L : 1;
            p[a].assign(n, nullptr);
            for (int l = 0; l < n; ++l) { p[a][l] = q; q += act_size(s, B, T, a); }
        }
    }
    R* operator()(int a, int l = 0) { return p[a][l]; }
};

// ----------------------------------------------------------------------------- layers, forward

// [torch-R] token/position embedding: x = wte[token] + wpe[position], positions 0..T-1.
template <class R>
static void encoder_forward(R* out, const int* inp, const R* wte, const R* wpe, int B, int T, int C) {
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t) {
            const R* we = wte + (int64_t)inp[b * T + t] * C;
            R* o = out + ((int64_t)b * T + t) * C;
            if (!wpe) {  // rotary position embedding: no learned position vector
                for (int c = 0; c < C; ++c) o[c] = we[c];
                continue;
            }
            const R* pe = wpe + (int64_t)t * C;
            for (int c = 0; c < C; ++c) o[c] = we[c] + pe[c];
        }
}

// [torch-R] Transformer block (nn_layer_norm, eps 1e-5): per row mean and biased
// variance over the C channels, y = (x - mean) / sqrt(var + eps) * w + b.
template <class R>
static void layernorm_forward(R* out, R* mean, R* rstd, const R* inp, const R* w, const R* b, int64_t N, int C) {
    const R eps = R(1e-5);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const R* x = inp + i * C;
        R m = 0;
        for (int c = 0; c < C; ++c) m += x[c];
        m /= C;
        R v = 0;
        for (int c = 0; c < C; ++c) { R d = x[c] - m; v += d * d; }
        v /= C;
        R r = R(1) / std::sqrt(v + eps);
        R* o = out + i * C;
        for (int c = 0; c < C; ++c) o[c] = (x[c] - m) * r * w[c] + b[c];
        mean[i] = m;
        rstd[i] = r;
    }
}

// RMSNorm (Llama-style block): y = x * rstd * w, rstd = 1 / sqrt(mean_c(x^2) + eps),
// eps = 1e-5 as for LayerNorm; mean[] is written as 0.
template <class R>
static void rmsnorm_forward(R* out, R* mean, R* rstd, const R* inp, const R* w, int64_t N, int C) {
    const R eps = R(1e-5);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const R* x = inp + i * C;
        R ms = 0;
        for (int c = 0; c < C; ++c) ms += x[c] * x[c];
        ms /= C;
        const R r = R(1) / std::sqrt(ms + eps);
        R* o = out + i * C;
        for (int c = 0; c < C; ++c) o[c] = x[c] * r * w[c];
        mean[i] = 0;
        rstd[i] = r;
    }
}

template <class R>
static inline R silu(R g) { return g / (R(1) + std::exp(-g)); }
// d silu / dg = sigma(g) (1 + g (1 - sigma(g)))
template <class R>
static inline R silu_grad(R g) {
    const R sg = R(1) / (R(1) + std::exp(-g));
    return sg * (R(1) + g * (R(1) - sg));
}

// SwiGLU: gu [N, 2H] holds (g_j, u_j) in columns 2j, 2j+1; out [N, H] = silu(g) * u.
template <class R>
static void swiglu_forward(R* out, const R* gu, int64_t N, int64_t H) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < H; ++j) {
            const R g = gu[i * 2 * H + 2 * j], u = gu[i * 2 * H + 2 * j + 1];
            out[i * H + j] = silu(g) * u;
        }
}

// Dot product with eight interleaved partial sums (a fixed summation order).
template <class R>
static inline R dot(const R* a, const R* b, int n) {
    R s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int k = 0;
    for (; k + 8 <= n; k += 8)
        for (int j = 0; j < 8; ++j) s[j] += a[k + j] * b[k + j];
    R acc = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
    for (; k < n; ++k) acc += a[k] * b[k];
    return acc;
}

// [c3000] ニューラルネットワーク層の実装: a linear layer is a matrix product plus a
// bias repeated over the rows.  Weights are (out, in) row-major: out = inp * w^T + bias.
template <class R>
static void matmul_forward(R* out, const R* inp, const R* w, const R* bias, int64_t N, int IC, int OC) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const R* x = inp + i * IC;
        R* o = out + i * OC;
        for (int j = 0; j < OC; ++j) o[j] = (bias ? bias[j] : R(0)) + dot(x, w + (int64_t)j * IC, IC);
    }
}

// ----------------------------------------------------------------------------- MX FP8 operands
// "fp16 and below" ([llm.c], the paragraph on what follows the CUDA port), read as OCP
// MXFP8 with E4M3 elements: blocks of 32 consecutive values along the reduction
// dimension share one scale 2^e, the smallest power of two with max|x| <= 448 * 2^e
// (nothing clips); each value becomes x / 2^e rounded to the nearest E4M3 value (ties
// to the even mantissa).  In MX mode a product's operand is its bf16 tensor (the
// configured storage precision, round-to-nearest-even) taken through this encoding and
// back; the product itself is the oracle's plain sum.

// Nearest bf16 value (round to nearest, ties to even) of a double, as the GPU stores it.
static double round_bf16(double v) {
    if (!std::isfinite(v) || v == 0.0) return v;
    int E;
    std::frexp(v, &E);                     // |v| in [2^(E-1), 2^E)
    const int ex = std::max(E - 1, -126);  // below 2^-126: bf16's subnormal spacing
    const double q = std::ldexp(1.0, ex - 7);
    return std::nearbyint(v / q) * q;      // v / q is exact; nearbyint rounds half to even
}

// Nearest E4M3 value of a scaled element (|a| <= 448 by the choice of scale): 3 mantissa
// bits below 2^-6 the fixed subnormal spacing 2^-9; ties to the even mantissa.
static double round_e4m3(double v) {
    const double a = std::fabs(v);
    if (a == 0.0) return v;
    if (a >= 448.0) return std::copysign(448.0, v);
    int E;
    std::frexp(a, &E);
    const int ex = std::max(E - 1, -6);
    const double q = std::ldexp(1.0, ex - 3);
    return std::copysign(std::nearbyint(a / q) * q, v);
}

// The block exponent: the smallest integer e with amax <= 448 * 2^e, within E8M0's
// [-127, 127]; an all-zero block takes -127.
static int mx_block_exponent(double amax) {
    if (!(amax > 0.0)) return -127;
    int p;
    std::frexp(amax, &p);              // floor(log2 amax) = p - 1
    int e = p - 1 - 8;                 // amax / 2^e in [256, 512)
    if (std::ldexp(amax, -e) > 448.0) ++e;
    return std::min(127, std::max(-127, e));
}

// y = the MX encoding of x [rows, K] taken back to real values (blocks of 32 along K;
// a last partial block reads as zero-padded), after rounding each x to bf16.
template <class R>
static void mx_roundtrip(R* y, const R* x, int64_t rows, int K) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int k0 = 0; k0 < K; k0 += 32) {
            const int k1 = std::min(K, k0 + 32);
            double v[32], amax = 0.0;
            for (int k = k0; k < k1; ++k) {
                v[k - k0] = round_bf16((double)x[r * K + k]);
                amax = std::max(amax, std::fabs(v[k - k0]));
            }
            const int e = mx_block_exponent(amax);
            for (int k = k0; k < k1; ++k)
                y[r * K + k] = (R)(std::ldexp(round_e4m3(std::ldexp(v[k - k0], -e)), e));
        }
}

// A linear layer whose two operands (in MX mode) go through the MX encoding first.
template <class R>
static void matmul_forward_mx(R* out, const R* inp, const R* w, const R* bias, int64_t N, int IC, int OC, bool mx) {
    if (!mx) return matmul_forward(out, inp, w, bias, N, IC, OC);
    std::vector<R> xq((size_t)N * IC), wq((size_t)OC * IC);
    mx_roundtrip(xq.data(), inp, N, IC);
    mx_roundtrip(wq.data(), w, OC, IC);
    matmul_forward(out, xq.data(), wq.data(), bias, N, IC, OC);
}

// [torch-R] 自注意力 and [nanogpt] 直觉上的self-attention / scaling:
// qkv columns are [q | k | v], each C wide, head h uses columns h*hs..(h+1)*hs-1;
// s_tu = q_t . k_u / sqrt(hs) for u <= t, softmax over u <= t (masked keys get
// weight exactly 0), y_t = sum_u a_tu v_u, heads side by side in y.
template <class R>
static void attention_forward(R* out, R* preatt, R* att, const R* qkv, int B, int T, int C, int NH) {
    const int hs = C / NH;
    const R scale = R(1) / std::sqrt(R(hs));
    const int64_t C3 = 3 * (int64_t)C;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < NH; ++h)
            for (int t = 0; t < T; ++t) {
                const R* q = qkv + ((int64_t)b * T + t) * C3 + h * hs;
                R* pre = preatt + (((int64_t)b * NH + h) * T + t) * T;
                R* a = att + (((int64_t)b * NH + h) * T + t) * T;
                R mx = -std::numeric_limits<R>::infinity();
                for (int u = 0; u <= t; ++u) {
                    const R* k = qkv + ((int64_t)b * T + u) * C3 + C + h * hs;
                    pre[u] = dot(q, k, hs) * scale;
                    if (pre[u] > mx) mx = pre[u];
                }
                R sum = 0;
                for (int u = 0; u <= t; ++u) { a[u] = std::exp(pre[u] - mx); sum += a[u]; }
                for (int u = 0; u <= t; ++u) a[u] /= sum;
                for (int u = t + 1; u < T; ++u) { pre[u] = -std::numeric_limits<R>::infinity(); a[u] = 0; }
                R* y = out + ((int64_t)b * T + t) * C + h * hs;
                for (int d = 0; d < hs; ++d) y[d] = 0;
                for (int u = 0; u <= t; ++u) {
                    const R* v = qkv + ((int64_t)b * T + u) * C3 + 2 * C + h * hs;
                    for (int d = 0; d < hs; ++d) y[d] += a[u] * v[d];
                }
            }
}

// GELU, tanh form printed in the [c3000] comment thread (and nn_gelu(approximate="tanh")
// in [torch-R] 前馈网络): g(x) = x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))).
template <class R>
static inline R gelu(R x) {
    const R k = (R)std::sqrt(2.0 / M_PI);
    return R(0.5) * x * (R(1) + std::tanh(k * (x + R(0.044715) * x * x * x)));
}
// Its derivative, by the product and chain rules.
template <class R>
static inline R gelu_grad(R x) {
    const R k = (R)std::sqrt(2.0 / M_PI);
    R u = k * (x + R(0.044715) * x * x * x);
    R th = std::tanh(u);
    R du = k * (R(1) + R(3) * R(0.044715) * x * x);
    return R(0.5) * (R(1) + th) + R(0.5) * x * (R(1) - th * th) * du;
}

template <class R>
static void gelu_forward(R* out, const R* inp, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = gelu(inp[i]);
}

template <class R>
static void residual_forward(R* out, const R* a, const R* b, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = a[i] + b[i];
}

// [nanogpt] 计算loss: cross-entropy of the next-token targets.  Per row the softmax
// probabilities (max-subtracted) and the loss logsumexp(z) - z[target].
template <class R>
static void softmax_crossentropy_forward(R* probs, R* losses, const R* logits, const int* targets, int64_t N, int V) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const R* z = logits + i * V;
        R* p = probs + i * V;
        R mx = z[0];
        for (int v = 1; v < V; ++v) if (z[v] > mx) mx = z[v];
        R sum = 0;
        for (int v = 0; v < V; ++v) sum += std::exp(z[v] - mx);
        R lse = mx + std::log(sum);
        for (int v = 0; v < V; ++v) p[v] = std::exp(z[v] - lse);
        if (targets) losses[i] = lse - z[targets[i]];
    }
}

// ----------------------------------------------------------------------------- layers, backward
// Each backward accumulates (+=) into its input gradients; the caller zeroes them.

template <class R>
static void encoder_backward(R* dwte, R* dwpe, const R* dout, const int* inp, int B, int T, int C) {
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t) {
            const R* d = dout + ((int64_t)b * T + t) * C;
            R* dw = dwte + (int64_t)inp[b * T + t] * C;
            for (int c = 0; c < C; ++c) dw[c] += d[c];
            if (!dwpe) continue;  // rotary: wpe is not used and keeps a zero gradient
            R* dp = dwpe + (int64_t)t * C;
            for (int c = 0; c < C; ++c) dp[c] += d[c];
        }
}

// LayerNorm backward, derived from y = xhat * w + b with xhat = (x - mean) * rstd:
//   dxhat = dy * w
//   dx    = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat))
//   dw    = sum_rows dy * xhat,   db = sum_rows dy
template <class R>
static void layernorm_backward(R* dinp, R* dw, R* db, const R* dout, const R* inp, const R* w,
                               const R* mean, const R* rstd, int64_t N, int C) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        const R* dy = dout + i * C;
        const R* x = inp + i * C;
        R m = mean[i], r = rstd[i];
        R s1 = 0, s2 = 0;
        for (int c = 0; c < C; ++c) {
            R xh = (x[c] - m) * r;
            R dxh = dy[c] * w[c];
            s1 += dxh;
            s2 += dxh * xh;
        }
        s1 /= C;
        s2 /= C;
        R* dx = dinp + i * C;
        for (int c = 0; c < C; ++c) {
            R xh = (x[c] - m) * r;
            R dxh = dy[c] * w[c];
            dx[c] += r * (dxh - s1 - xh * s2);
        }
    }
#pragma omp parallel for schedule(static)
    for (int c = 0; c < C; ++c) {
        R sw = 0, sb = 0;
        for (int64_t i = 0; i < N; ++i) {
            R xh = (inp[i * C + c] - mean[i]) * rstd[i];
            sw += dout[i * C + c] * xh;
            sb += dout[i * C + c];
        }
        dw[c] += sw;
        db[c] += sb;
    }
}

// Linear backward for out = inp * w^T + bias:
//   dinp = dout * w,  dw = dout^T * inp,  dbias = column sums of dout.
// RMSNorm backward, from y = xhat * w with xhat = x * rstd:
//   dxhat = dy * w,  dx = rstd * (dxhat - xhat * mean_c(dxhat * xhat)),  dw = sum_rows dy * xhat
template <class R>
static void rmsnorm_backward(R* dinp, R* dw, const R* dout, const R* inp, const R* w, const R* rstd, int64_t N,
                             int C) {
    for (int64_t i = 0; i < N; ++i) {
        const R* dy = dout + i * C;
        const R* x = inp + i * C;
        const R r = rstd[i];
        R m = 0;
        for (int c = 0; c < C; ++c) m += dy[c] * w[c] * x[c] * r;
        m /= C;
        R* dx = dinp + i * C;
        for (int c = 0; c < C; ++c) {
            const R xh = x[c] * r;
            dx[c] += r * (dy[c] * w[c] - xh * m);
            dw[c] += dy[c] * xh;
        }
    }
}

// SwiGLU backward: dg = dh u silu'(g), du = dh silu(g), into the interleaved columns.
template <class R>
static void swiglu_backward(R* dgu, const R* dout, const R* gu, int64_t N, int64_t H) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i)
        for (int64_t j = 0; j < H; ++j) {
            const R g = gu[i * 2 * H + 2 * j], u = gu[i * 2 * H + 2 * j + 1], dh = dout[i * H + j];
            dgu[i * 2 * H + 2 * j] += dh * u * silu_grad(g);
            dgu[i * 2 * H + 2 * j + 1] += dh * silu(g);
        }
}

// Input gradient of a linear layer: dinp [N, IC] += dout [N, OC] w [OC, IC].
template <class R>
static void matmul_backward_input(R* dinp, const R* dout, const R* w, int64_t N, int IC, int OC) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        R* dx = dinp + i * IC;
        const R* dy = dout + i * OC;
        for (int j = 0; j < OC; ++j) {
            const R g = dy[j];
            const R* wr = w + (int64_t)j * IC;
            for (int k = 0; k < IC; ++k) dx[k] += g * wr[k];
        }
    }
}

// The same with both operands taken through the MX encoding along the contraction
// (OC): dout's rows in blocks of 32 outputs, and for every input feature k the column
// w[:, k] in blocks of 32 outputs -- the rows of w^T, the layout a matrix core takes.
template <class R>
static void matmul_backward_input_mx(R* dinp, const R* dout, const R* w, int64_t N, int IC, int OC) {
    std::vector<R> dq((size_t)N * OC), wt((size_t)IC * OC), wtq((size_t)IC * OC), wq((size_t)OC * IC);
    mx_roundtrip(dq.data(), dout, N, OC);
    for (int j = 0; j < OC; ++j)
        for (int k = 0; k < IC; ++k) wt[(size_t)k * OC + j] = w[(size_t)j * IC + k];
    mx_roundtrip(wtq.data(), wt.data(), IC, OC);
    for (int j = 0; j < OC; ++j)
        for (int k = 0; k < IC; ++k) wq[(size_t)j * IC + k] = wtq[(size_t)k * OC + j];
    matmul_backward_input(dinp, dq.data(), wq.data(), N, IC, OC);
}

template <class R>
static void matmul_backward(R* dinp, R* dw, R* dbias, const R* dout, const R* inp, const R* w,
                            int64_t N, int IC, int OC, bool mx_dx = false) {
    if (mx_dx) matmul_backward_input_mx(dinp, dout, w, N, IC, OC);
    else matmul_backward_input(dinp, dout, w, N, IC, OC);
#pragma omp parallel for schedule(static)
    for (int j = 0; j < OC; ++j) {
        R* dwr = dw + (int64_t)j * IC;
        R sb = 0;
        for (int64_t i = 0; i < N; ++i) {
            const R g = dout[i * OC + j];
            const R* x = inp + i * IC;
            for (int k = 0; k < IC; ++k) dwr[k] += g * x[k];
            sb += g;
        }
        if (dbias) dbias[j] += sb;
    }
}

// Attention backward (softmax Jacobian; masked weights are 0 and stay 0):
//   da_tu = dy_t . v_u,  dv_u += a_tu dy_t
//   ds_tu = a_tu (da_tu - sum_u' a_tu' da_tu')
//   dq_t += sum_u ds_tu k_u / sqrt(hs),  dk_u += sum_t ds_tu q_t / sqrt(hs)
template <class R>
static void attention_backward(R* dqkv, R* dpreatt, R* datt, const R* dout, const R* qkv, const R* att,
                               int B, int T, int C, int NH) {
    const int hs = C / NH;
    const R scale = R(1) / std::sqrt(R(hs));
    const int64_t C3 = 3 * (int64_t)C;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < NH; ++h) {
            for (int t = 0; t < T; ++t) {
                const R* a = att + (((int64_t)b * NH + h) * T + t) * T;
                R* da = datt + (((int64_t)b * NH + h) * T + t) * T;
                R* ds = dpreatt + (((int64_t)b * NH + h) * T + t) * T;
                const R* dy = dout + ((int64_t)b * T + t) * C + h * hs;
                for (int u = 0; u <= t; ++u) {
                    const R* v = qkv + ((int64_t)b * T + u) * C3 + 2 * C + h * hs;
                    R* dv = dqkv + ((int64_t)b * T + u) * C3 + 2 * C + h * hs;
                    da[u] = dot(dy, v, hs);
                    for (int d = 0; d < hs; ++d) dv[d] += a[u] * dy[d];
                }
                R s = 0;
                for (int u = 0; u <= t; ++u) s += a[u] * da[u];
                for (int u = 0; u <= t; ++u) ds[u] = a[u] * (da[u] - s);
                const R* q = qkv + ((int64_t)b * T + t) * C3 + h * hs;
                R* dq = dqkv + ((int64_t)b * T + t) * C3 + h * hs;
                for (int u = 0; u <= t; ++u) {
                    const R* k = qkv + ((int64_t)b * T + u) * C3 + C + h * hs;
                    R* dk = dqkv + ((int64_t)b * T + u) * C3 + C + h * hs;
                    for (int d = 0; d < hs; ++d) {
                        dq[d] += ds[u] * scale * k[d];
                        dk[d] += ds[u] * scale * q[d];
                    }
                }
            }
        }
}

template <class R>
static void gelu_backward(R* dinp, const R* inp, const R* dout, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) dinp[i] += gelu_grad(inp[i]) * dout[i];
}

// d(mean loss)/dz = (softmax(z) - onehot(target)) / (B*T).
template <class R>
static void crossentropy_softmax_backward(R* dlogits, const R* probs, const int* targets, int64_t N, int V) {
    const R inv = R(1) / R(N);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N; ++i) {
        R* d = dlogits + i * V;
        const R* p = probs + i * V;
        for (int v = 0; v < V; ++v) d[v] += p[v] * inv;
        d[targets[i]] -= inv;
    }
}

// ----------------------------------------------------------------------------- rotary position embedding
// RoFormer's rotary position embedding (named in "GPT-2 from scratch with torch", token
// and position embedding, as the newer alternative to learned position vectors, after
// Su et al. 2021): a head vector x at position m has each pair (x[2i], x[2i+1]) turned
// by the angle m * theta_i, theta_i = base^(-2i / hs):
//   x'[2i]   = x[2i] cos(m theta_i) - x[2i+1] sin(m theta_i)
//   x'[2i+1] = x[2i] sin(m theta_i) + x[2i+1] cos(m theta_i)
// Applied to the query and key heads (not the values) before the scores.  The
// backward pass turns the gradients back by -m theta_i (a rotation's transpose).
// Angles are taken in double whatever R is.
template <class R>
static void rope_head(R* out, const R* x, int hs, int m, double base, int sign) {
    for (int i = 0; i < hs / 2; ++i) {
        const double th = std::pow(base, -2.0 * i / hs), a = sign * (double)m * th;
        const double c = std::cos(a), sn = std::sin(a);
        const double x0 = x[2 * i], x1 = x[2 * i + 1];
        out[2 * i] = (R)(x0 * c - x1 * sn);
        out[2 * i + 1] = (R)(x0 * sn + x1 * c);
    }
}

// qkv [B*T, 3C] (q | k | v, head h at columns h*hs of each third) -> out with q and k
// of every head turned for its position t; v copied.  sign -1: the inverse turn.
template <class R>
static void rope_qkv(R* out, const R* qkv, int B, int T, int C, int NH, double base, int sign) {
    const int hs = C / NH;
    const int64_t C3 = 3 * (int64_t)C;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t) {
            const R* x = qkv + ((int64_t)b * T + t) * C3;
            R* o = out + ((int64_t)b * T + t) * C3;
            for (int h = 0; h < 2 * NH; ++h) rope_head(o + h * hs, x + h * hs, hs, t, base, sign);
            for (int c = 2 * C; c < 3 * C; ++c) o[c] = x[c];
        }
}

// ----------------------------------------------------------------------------- model

struct ModelBase {
    virtual ~ModelBase() {}
    Shape s;
    int B = 0, T = 0;
    int prec = 0;
};

template <class R>
struct Model : ModelBase {
    std::vector<R> params, grads, m, v;
    Params<R> P, G;
    Acts<R> A, dA;
    std::vector<int> inputs, targets;
    bool have_targets = false, have_forward = false;
    R loss = -1;
    // rotary position embedding (off: learned wpe).  qkv_rot[l]: the attention's
    // q | k | v with q and k turned; outside the plain activation set.
    bool rotary = false;
    double rope_base = 10000.0;
    // MX FP8 operands for the forward pass's block and lm_head products (the backward
    // pass uses the stored activations and weights as they are: straight-through);
    // mx_dx: also for the input-gradient products of those layers in the backward pass
    // (the weight gradients keep the plain operands)
    bool mx = false, mx_dx = false;
    std::vector<std::vector<R>> qkv_rot;
    std::vector<R> dqkv_rot;

    Model(const Shape& sh, int b, int t) {
        s = sh; B = b; T = t;
        int64_t n = count_params(s);
        params.assign(n, R(0)); grads.assign(n, R(0)); m.assign(n, R(0)); v.assign(n, R(0));
        P.bind(params.data(), s);
        G.bind(grads.data(), s);
        A.alloc(s, B, T);
        inputs.assign((size_t)B * T, 0);
        targets.assign((size_t)B * T, 0);
    }

    // [llm.c] forward: encoder, L pre-norm blocks, final LN, tied logits, softmax, cross-entropy.
    // Block structure per [torch-R] Transformer block: x = x + attn(ln_1(x)); x = x + mlp(ln_2(x)).
    void forward(const int* inp, const int* tgt) {
        const int C = s.C, L = s.L, NH = s.NH, V = s.V;
        const int64_t BT = (int64_t)B * T;
        std::memcpy(inputs.data(), inp, sizeof(int) * BT);
        have_targets = tgt != nullptr;
        if (tgt) std::memcpy(targets.data(), tgt, sizeof(int) * BT);
        const bool llama = s.block == 1;
        const int64_t H = llama_hidden(C);
        auto bias = [&](int k, int l) -> const R* { return llama ? nullptr : P.t[k][l]; };
        auto norm = [&](R* out, R* mean, R* rstd, const R* x, const R* w, const R* b) {
            if (llama) rmsnorm_forward(out, mean, rstd, x, w, BT, C);
            else layernorm_forward(out, mean, rstd, x, w, b, BT, C);
        };
        encoder_forward(A(A_ENCODED), inp, P.wte, rotary ? (const R*)nullptr : P.wpe, B, T, C);
        if (rotary) qkv_rot.assign(L, std::vector<R>((size_t)3 * BT * C));
        for (int l = 0; l < L; ++l) {
            const R* x = l == 0 ? A(A_ENCODED) : A(A_RESIDUAL3, l - 1);
            norm(A(A_LN1, l), A(A_LN1_MEAN, l), A(A_LN1_RSTD, l), x, P.t[LN1W][l], P.t[LN1B][l]);
            matmul_forward_mx(A(A_QKV, l), A(A_LN1, l), P.t[QKVW][l], bias(QKVB, l), BT, C, 3 * C, mx);
            const R* qkv = A(A_QKV, l);
            if (rotary) {
                rope_qkv(qkv_rot[l].data(), A(A_QKV, l), B, T, C, NH, rope_base, +1);
                qkv = qkv_rot[l].data();
            }
            attention_forward(A(A_ATTY, l), A(A_PREATT, l), A(A_ATT, l), qkv, B, T, C, NH);
            matmul_forward_mx(A(A_ATTPROJ, l), A(A_ATTY, l), P.t[PROJW][l], bias(PROJB, l), BT, C, C, mx);
            residual_forward(A(A_RESIDUAL2, l), x, A(A_ATTPROJ, l), BT * C);
            norm(A(A_LN2, l), A(A_LN2_MEAN, l), A(A_LN2_RSTD, l), A(A_RESIDUAL2, l), P.t[LN2W][l], P.t[LN2B][l]);
            if (llama) {
                matmul_forward(A(A_FCH, l), A(A_LN2, l), P.t[FCW][l], (const R*)nullptr, BT, C, (int)(2 * H));
                swiglu_forward(A(A_FCH_GELU, l), A(A_FCH, l), BT, H);
                matmul_forward(A(A_FCPROJ, l), A(A_FCH_GELU, l), P.t[FCPW][l], (const R*)nullptr, BT, (int)H, C);
            } else {
                matmul_forward_mx(A(A_FCH, l), A(A_LN2, l), P.t[FCW][l], P.t[FCB][l], BT, C, 4 * C, mx);
                gelu_forward(A(A_FCH_GELU, l), A(A_FCH, l), BT * 4 * C);
                matmul_forward_mx(A(A_FCPROJ, l), A(A_FCH_GELU, l), P.t[FCPW][l], P.t[FCPB][l], BT, 4 * C, C, mx);
            }
            residual_forward(A(A_RESIDUAL3, l), A(A_RESIDUAL2, l), A(A_FCPROJ, l), BT * C);
        }
        const R* xL = A(A_RESIDUAL3, L - 1);
        norm(A(A_LNF), A(A_LNF_MEAN), A(A_LNF_RSTD), xL, P.lnfw, P.lnfb);
        // [c3000] Transformer本体 / [torch-R] 输出: logits = final hidden state times the
        // token-embedding matrix (tied lm_head, no bias).
        matmul_forward_mx(A(A_LOGITS), A(A_LNF), P.wte, (const R*)nullptr, BT, C, V, mx);
        softmax_crossentropy_forward(A(A_PROBS), A(A_LOSSES), A(A_LOGITS), tgt, BT, V);
        if (tgt) {
            R acc = 0;
            for (int64_t i = 0; i < BT; ++i) acc += A(A_LOSSES)[i];
            loss = acc / R(BT);
        } else {
            loss = -1;
        }
        have_forward = true;
    }

    // Reverse of forward; parameter gradients are overwritten (zeroed first).
    int backward() {
        if (!have_forward || !have_targets) return -4;
        const int C = s.C, L = s.L, NH = s.NH, V = s.V;
        const int64_t BT = (int64_t)B * T;
        if (dA.mem.empty()) dA.alloc(s, B, T);
        std::fill(grads.begin(), grads.end(), R(0));
        std::fill(dA.mem.begin(), dA.mem.end(), R(0));
        crossentropy_softmax_backward(dA(A_LOGITS), A(A_PROBS), targets.data(), BT, V);
        const bool llama = s.block == 1;
        const int64_t H = llama_hidden(C);
        auto gbias = [&](int k, int l) -> R* { return llama ? nullptr : G.t[k][l]; };
        auto norm_bwd = [&](R* dx, R* dw, R* db, const R* dy, const R* x, const R* w, const R* mean, const R* rstd) {
            if (llama) rmsnorm_backward(dx, dw, dy, x, w, rstd, BT, C);
            else layernorm_backward(dx, dw, db, dy, x, w, mean, rstd, BT, C);
        };
        matmul_backward(dA(A_LNF), G.wte, (R*)nullptr, dA(A_LOGITS), A(A_LNF), P.wte, BT, C, V, mx_dx);
        R* dxL = dA(A_RESIDUAL3, L - 1);
        norm_bwd(dxL, G.lnfw, G.lnfb, dA(A_LNF), A(A_RESIDUAL3, L - 1), P.lnfw, A(A_LNF_MEAN), A(A_LNF_RSTD));
        for (int l = L - 1; l >= 0; --l) {
            const R* x = l == 0 ? A(A_ENCODED) : A(A_RESIDUAL3, l - 1);
            R* dx = l == 0 ? dA(A_ENCODED) : dA(A_RESIDUAL3, l - 1);
            R* dres3 = dA(A_RESIDUAL3, l);
            // residual3 = residual2 + fcproj: the gradient reaches both unchanged
            R* dres2 = dA(A_RESIDUAL2, l);
            for (int64_t i = 0; i < BT * C; ++i) { dres2[i] += dres3[i]; dA(A_FCPROJ, l)[i] += dres3[i]; }
            if (llama) {
                matmul_backward(dA(A_FCH_GELU, l), G.t[FCPW][l], (R*)nullptr, dA(A_FCPROJ, l), A(A_FCH_GELU, l),
                                P.t[FCPW][l], BT, (int)H, C);
                swiglu_backward(dA(A_FCH, l), dA(A_FCH_GELU, l), A(A_FCH, l), BT, H);
                matmul_backward(dA(A_LN2, l), G.t[FCW][l], (R*)nullptr, dA(A_FCH, l), A(A_LN2, l), P.t[FCW][l], BT, C,
                                (int)(2 * H));
            } else {
                matmul_backward(dA(A_FCH_GELU, l), G.t[FCPW][l], G.t[FCPB][l], dA(A_FCPROJ, l), A(A_FCH_GELU, l),
                                P.t[FCPW][l], BT, 4 * C, C, mx_dx);
                gelu_backward(dA(A_FCH, l), A(A_FCH, l), dA(A_FCH_GELU, l), BT * 4 * C);
                matmul_backward(dA(A_LN2, l), G.t[FCW][l], G.t[FCB][l], dA(A_FCH, l), A(A_LN2, l), P.t[FCW][l], BT, C,
                                4 * C, mx_dx);
            }
            norm_bwd(dres2, G.t[LN2W][l], G.t[LN2B][l], dA(A_LN2, l), A(A_RESIDUAL2, l), P.t[LN2W][l],
                     A(A_LN2_MEAN, l), A(A_LN2_RSTD, l));
            // residual2 = x + attproj
            for (int64_t i = 0; i < BT * C; ++i) { dx[i] += dres2[i]; dA(A_ATTPROJ, l)[i] += dres2[i]; }
            matmul_backward(dA(A_ATTY, l), G.t[PROJW][l], gbias(PROJB, l), dA(A_ATTPROJ, l), A(A_ATTY, l),
                            P.t[PROJW][l], BT, C, C, mx_dx && !llama);
            if (rotary) {
                // gradients reach the turned q | k | v, then turn back to the qkv product's output
                dqkv_rot.assign((size_t)3 * BT * C, R(0));
                attention_backward(dqkv_rot.data(), dA(A_PREATT, l), dA(A_ATT, l), dA(A_ATTY, l), qkv_rot[l].data(),
                                   A(A_ATT, l), B, T, C, NH);
                rope_qkv(dA(A_QKV, l), dqkv_rot.data(), B, T, C, NH, rope_base, -1);
            } else {
                attention_backward(dA(A_QKV, l), dA(A_PREATT, l), dA(A_ATT, l), dA(A_ATTY, l), A(A_QKV, l),
                                   A(A_ATT, l), B, T, C, NH);
            }
            matmul_backward(dA(A_LN1, l), G.t[QKVW][l], gbias(QKVB, l), dA(A_QKV, l), A(A_LN1, l), P.t[QKVW][l], BT, C,
                            3 * C, mx_dx && !llama);
            norm_bwd(dx, G.t[LN1W][l], G.t[LN1B][l], dA(A_LN1, l), x, P.t[LN1W][l], A(A_LN1_MEAN, l),
                     A(A_LN1_RSTD, l));
        }
        encoder_backward(G.wte, rotary ? (R*)nullptr : G.wpe, dA(A_ENCODED), inputs.data(), B, T, C);
        return 0;
    }

    // [llm.c] Adam update; decoupled weight decay (AdamW) with bias correction, t from 1:
    //   m = b1 m + (1-b1) g,  v = b2 v + (1-b2) g^2,
    //   theta -= lr * ( (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) + wd * theta ).
    void adamw(R lr, R b1, R b2, R eps, R wd, int t) {
        const R c1 = R(1) - std::pow(b1, (R)t);
        const R c2 = R(1) - std::pow(b2, (R)t);
        const int64_t n = (int64_t)params.size();
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i) {
            R g = grads[i];
            m[i] = b1 * m[i] + (R(1) - b1) * g;
            v[i] = b2 * v[i] + (R(1) - b2) * g * g;
            R mh = m[i] / c1;
            R vh = v[i] / c2;
            params[i] -= lr * (mh / (std::sqrt(vh) + eps) + wd * params[i]);
        }
    }

    std::vector<R>* vec(const char* name) {
        if (!strcmp(name, "params")) return &params;
        if (!strcmp(name, "grads")) return &grads;
        if (!strcmp(name, "m")) return &m;
        if (!strcmp(name, "v")) return &v;
        return nullptr;
    }

    // Activation ("name") or activation gradient ("dname") pointer and size.
    R* act(const char* name, int layer, int64_t* n) {
        if (!strcmp(name, "qkv_rot")) {  // rotary mode, after a forward pass
            if (layer < 0 || layer >= (int)qkv_rot.size()) return nullptr;
            *n = (int64_t)qkv_rot[layer].size();
            return qkv_rot[layer].data();
        }
        bool grad = name[0] == 'd' && strcmp(name, "d") != 0;
        const char* nm = grad ? name + 1 : name;
        for (int a = 0; a < NACT; ++a)
            if (!strcmp(nm, kActNames[a])) {
                int nl = act_per_layer(a) ? s.L : 1;
                if (layer < 0 || layer >= nl) return nullptr;
                if (grad && dA.mem.empty()) return nullptr;
                *n = act_size(s, B, T, a);
                return grad ? dA(a, layer) : A(a, layer);
            }
        return nullptr;
    }
};

thread_local std::string g_err;

}  // namespace

// ============================================================================= C API (ctypes)
extern "C" {

const char* orc_last_error() { return g_err.c_str(); }

int64_t orc_num_parameters(int V, int P, int L, int NH, int C) { return count_params(Shape{V, P, L, NH, C}); }

int64_t orc_num_activations(int V, int P, int L, int NH, int C, int B, int T) {
    return count_acts(Shape{V, P, L, NH, C}, B, T);
}

// prec: 0 = float, 1 = double.  Returns NULL on invalid shapes or allocation failure.
// block: 0 GPT-2, 1 Llama-style (which always uses the rotary position embedding).
void* orc_create_block(int prec, int V, int P, int L, int NH, int C, int B, int T, int block) {
    if (V < 1 || P < 1 || L < 1 || NH < 1 || C < 1 || C % NH || B < 1 || T < 1 || T > P || block < 0 || block > 1) {
        g_err = "invalid shape";
        return nullptr;
    }
    Shape s{V, P, L, NH, C, block};
    try {
        if (prec == 0) { auto* m = new Model<float>(s, B, T); m->prec = 0; m->rotary = block == 1; return m; }
        if (prec == 1) { auto* m = new Model<double>(s, B, T); m->prec = 1; m->rotary = block == 1; return m; }
    } catch (const std::bad_alloc&) {
        g_err = "out of host memory";
        return nullptr;
    }
    g_err = "prec must be 0 or 1";
    return nullptr;
}

void* orc_create(int prec, int V, int P, int L, int NH, int C, int B, int T) {
    return orc_create_block(prec, V, P, L, NH, C, B, T, 0);
}

int64_t orc_num_parameters_block(int V, int P, int L, int NH, int C, int block) {
    return count_params(Shape{V, P, L, NH, C, block});
}

void orc_silu(const double* x, double* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = silu(x[i]); }
void orc_silu_grad(const double* x, double* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = silu_grad(x[i]); }

void orc_destroy(void* h) { delete (ModelBase*)h; }

#define ORC_DISPATCH(h, EXPR)                                              \
    do {                                                                   \
        ModelBase* mb__ = (ModelBase*)(h);                                 \
        if (mb__->prec == 0) { auto* M = (Model<float>*)mb__; EXPR; }      \
        else { auto* M = (Model<double>*)mb__; EXPR; }                     \
    } while (0)

// name in {params, grads, m, v}; copies n values from/to double arrays.
int orc_set_vec(void* h, const char* name, const double* src, int64_t n) {
    int rc = 0;
    ORC_DISPATCH(h, {
        auto* v = M->vec(name);
        if (!v || (int64_t)v->size() != n) { g_err = "bad vector name or size"; rc = -1; }
        else { using R = typename std::decay<decltype((*v)[0])>::type; for (int64_t i = 0; i < n; ++i) (*v)[i] = (R)src[i]; }
    });
    return rc;
}
int orc_set_vec_f32(void* h, const char* name, const float* src, int64_t n) {
    int rc = 0;
    ORC_DISPATCH(h, {
        auto* v = M->vec(name);
        if (!v || (int64_t)v->size() != n) { g_err = "bad vector name or size"; rc = -1; }
        else for (int64_t i = 0; i < n; ++i) (*v)[i] = src[i];
    });
    return rc;
}
int orc_get_vec(void* h, const char* name, double* dst, int64_t n) {
    int rc = 0;
    ORC_DISPATCH(h, {
        auto* v = M->vec(name);
        if (!v || (int64_t)v->size() != n) { g_err = "bad vector name or size"; rc = -1; }
        else for (int64_t i = 0; i < n; ++i) dst[i] = (double)(*v)[i];
    });
    return rc;
}

int64_t orc_act_numel(void* h, const char* name, int layer) {
    int64_t n = -1;
    ORC_DISPATCH(h, { if (!M->act(name, layer, &n)) n = -1; });
    return n;
}
int orc_get_act(void* h, const char* name, int layer, double* dst, int64_t n) {
    int rc = 0;
    ORC_DISPATCH(h, {
        int64_t k = 0;
        auto* p = M->act(name, layer, &k);
        if (!p || k != n) { g_err = "bad activation name, layer or size"; rc = -1; }
        else for (int64_t i = 0; i < n; ++i) dst[i] = (double)p[i];
    });
    return rc;
}

// targets may be NULL (then no loss).  Returns the mean loss, or -1 without targets.
double orc_forward(void* h, const int* inputs, const int* targets) {
    double out = -1;
    ModelBase* mb = (ModelBase*)h;
    const int64_t BT = (int64_t)mb->B * mb->T;
    for (int64_t i = 0; i < BT; ++i)
        if (inputs[i] < 0 || inputs[i] >= mb->s.V || (targets && (targets[i] < 0 || targets[i] >= mb->s.V))) {
            g_err = "token id out of range";
            return std::numeric_limits<double>::quiet_NaN();
        }
    ORC_DISPATCH(h, { M->forward(inputs, targets); out = (double)M->loss; });
    return out;
}

// Rotary position embedding on (1) or off (0, learned wpe) for the following passes.
int orc_set_rotary(void* h, int on, double base) {
    if (!(base > 1.0)) { g_err = "rotary base must exceed 1"; return -1; }
    if (!on && ((ModelBase*)h)->s.block == 1) { g_err = "the Llama-style block always uses rotary positions"; return -1; }
    ORC_DISPATCH(h, { M->rotary = on != 0; M->rope_base = base; M->have_forward = false; M->qkv_rot.clear(); });
    return 0;
}

// MX FP8 operands: 0 off, 1 for the forward pass's block and lm_head products, 2 for
// those and for the backward pass's input-gradient products of the same layers.
int orc_set_mx(void* h, int mode) {
    if (((ModelBase*)h)->s.block != 0) { g_err = "MX products are modelled for the GPT-2 block"; return -1; }
    if (mode < 0 || mode > 2) { g_err = "MX mode must be 0, 1 or 2"; return -1; }
    ORC_DISPATCH(h, { M->mx = mode >= 1; M->mx_dx = mode == 2; M->have_forward = false; });
    return 0;
}

// dinp [N, IC] = dout [N, OC] w [OC, IC] with both operands through bf16 and the MX
// encoding along OC (float64).
void orc_matmul_backward_input_mx(const double* dout, const double* w, int64_t N, int IC, int OC, double* dinp) {
    std::fill(dinp, dinp + N * IC, 0.0);
    matmul_backward_input_mx(dinp, dout, w, N, IC, OC);
}

// y = x [rows, K] taken through bf16 and the MX FP8 encoding and back (float64).
void orc_mx_roundtrip(const double* x, double* y, int64_t rows, int K) { mx_roundtrip(y, x, rows, K); }

// y[r] = x[r] (one head vector of hs values) turned for position pos[r]; inverse turns back.
void orc_rope(const double* x, double* y, int rows, int hs, const int* pos, double base, int inverse) {
    for (int r = 0; r < rows; ++r) rope_head(y + (int64_t)r * hs, x + (int64_t)r * hs, hs, pos[r], base, inverse ? -1 : 1);
}

int orc_backward(void* h) {
    int rc = 0;
    ORC_DISPATCH(h, { rc = M->backward(); });
    if (rc) g_err = "backward needs a prior forward with targets";
    return rc;
}

int orc_adamw(void* h, double lr, double b1, double b2, double eps, double wd, int t) {
    if (t < 1) { g_err = "step must be >= 1"; return -1; }
    ORC_DISPATCH(h, { using R = std::remove_reference_t<decltype(M->params[0])>;
                      M->adamw((R)lr, (R)b1, (R)b2, (R)eps, (R)wd, t); });
    return 0;
}

// Element-wise GELU (tanh form) and its derivative, float64, for pin tests.
void orc_gelu(const double* x, double* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = gelu(x[i]); }
void orc_gelu_grad(const double* x, double* y, int64_t n) { for (int64_t i = 0; i < n; ++i) y[i] = gelu_grad(x[i]); }

int orc_num_threads() {
#ifdef _OPENMP
    int n = 0;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    return 1;
#endif
}

// Threads for the loops that follow (the CPU-baseline timing runs at two counts);
// results do not depend on it.
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

}  // extern "C"
