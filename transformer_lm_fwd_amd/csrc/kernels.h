// Launch wrappers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace gpt2 {

// Sets the message gpt2_last_error() returns and returns `code` (host code of the library).
int report_error(int code, const char* msg);

// Records the launch(es) in its lifetime when the launch profiler is on.
// True while the launch profiler records (the backward pass then runs on one
// stream so that overlapping launches do not inflate each other's durations).
bool profiling();

struct ProfScope {
    ProfScope(hipStream_t s, const char* name, double flops, double bytes);
    ~ProfScope();
    int idx;
    hipStream_t stream;
};

// ---------------------------------------------------------------- GEMM
// C[m, n] = epilogue( sum_k A(m, k) * B(n, k) ), fp32 accumulation on MFMA.
// A(m, k) = A[m*lda + k] when a_kcontig, else A[k*lda + m]; likewise B(n, k).
enum GemmEpi {
    EPI_BIAS = 0,       // C = acc + bias[n]            (bias may be null)
    EPI_BIAS_RES = 1,   // C = R[m, n] + acc + bias[n]  (R has row stride ldc)
    EPI_BIAS_GELU = 2,  // C = acc + bias[n], C2 = gelu(C)
    EPI_GELU_BWD = 3,   // C = acc * gelu'(R[m, n])
    EPI_F32 = 4         // fp32 C = acc (split-K partials or a direct fp32 result)
};

struct GemmArgs {
    const void* A;
    const void* B;
    void* C;
    void* C2;
    const void* R;
    const float* bias;
    // EPI_F32 with an m-contiguous A (bf16 only): if non-null, also receives the row
    // sums of op(A) over k, rowsum[m] = sum_k op(A)[m, k] (fp32, overwritten) - the
    // bias gradient of a weight-gradient product dW = dY^T X.
    float* rowsum;
    int M, N, K;
    int64_t lda, ldb, ldc;
    // MX FP8 operands (gemm_mx only): E8M0 block scales of A and B, laid out
    // [K / 128][rows][4] bytes (byte j of row r's word in k-stage t: the scale of
    // k-block 4 t + j), with srows_a / srows_b rows per k-stage.
    const uint8_t* sa;
    const uint8_t* sb;
    int64_t srows_a, srows_b;
    // EPI_BIAS_GELU with q2 non-null (N a multiple of 128, bf16 output): also the MX
    // codes of the bf16 GELU output, q2 [M, N] (row stride ldq2 bytes), and their
    // scales s2 [N / 128][M][4] - the input of a following MX product.
    uint8_t* q2;
    uint8_t* s2;
    int64_t ldq2;
    // EPI_BIAS extras of the bf16 (and MX) products, each off when null:
    //  rope: turn the pairs of columns < rope_cols (whole heads of rope_hs) of row m by
    //        the (cos, sin) row of position m % rope_period (the rotary embedding);
    //  swiglu: columns (2j, 2j+1) are (gate, up) of hidden unit j: also write
    //        silu(gate) * up (from the bf16-rounded pair) to swiglu[m * ld_swiglu + j].
    //  swiglu_gu (backward): the product is dh; instead of storing it, read the (gate, up)
    //        pairs of hidden units j from swiglu_gu[m * 2 ld_swiglu + 2j, + 1] and write
    //        (dh u silu'(g), dh silu(g)) to swiglu[m * 2 ld_swiglu + 2j, + 1].
    const float2* rope;
    int rope_period, rope_hs, rope_cols;
    bf16* swiglu;
    int64_t ld_swiglu;
    const bf16* swiglu_gu;
};

// Returns hipSuccess or the launch error.  T in {float, bf16}: operand type;
// outputs of EPI_BIAS..EPI_GELU_BWD are T, EPI_F32 writes fp32.
template <class T>
hipError_t gemm(const GemmArgs& a, bool a_kcontig, bool b_kcontig, int epi, float* splitk_ws,
                size_t splitk_ws_floats, hipStream_t s);

// ---------------------------------------------------------------- element-wise / row kernels
template <class T>
hipError_t encoder_forward(T* out, const int32_t* tok, const float* wte, const float* wpe, int BT, int T_, int C,
                           hipStream_t s, int pos0 = 0);
template <class T>
// bf16 only: mxq / mxs non-null also write the output's MX FP8 codes [N, Kp] (row
// stride ldq bytes, Kp = C rounded up to 128) and scales [Kp / 128][N][4].
// rms: RMSNorm (mean taken as 0, statistics (0, rstd)); b may be null.
hipError_t layernorm_forward(T* out, float* stats, const T* inp, const float* w, const float* b, int N, int C,
                             hipStream_t s, uint8_t* mxq = nullptr, int64_t ldq = 0, uint8_t* mxs = nullptr,
                             bool rms = false);
// dres = dres_in + LN backward dx (dres_in may be null, or equal to dres); dw, db
// (overwrite) from column sums through `partial`.
template <class T>
hipError_t layernorm_backward(T* dres, const T* dres_in, float* dw, float* db, const T* dout, const T* inp,
                              const float* stats, const float* w, int N, int C, float* partial, size_t partial_floats,
                              hipStream_t s, bool rms = false, uint8_t* q = nullptr, int64_t ldq = 0,
                              uint8_t* sc = nullptr);  // rms: RMSNorm, db may be null; q: MX codes of dres (bf16)
// The two halves of layernorm_backward, for callers that run them on different streams.
template <class T>
hipError_t layernorm_backward_dx(T* dres, const T* dres_in, const T* dout, const T* inp, const float* stats,
                                 const float* w, int N, int C, hipStream_t s, bool rms = false);
template <class T>
hipError_t layernorm_param_grads(float* dw, float* db, const T* dout, const T* inp, const float* stats, int N, int C,
                                 float* partial, size_t partial_floats, hipStream_t s);
// dbias[n] = sum_m dout[m, n] (overwrite), deterministic two-stage.
template <class T>
hipError_t bias_grad(float* dbias, const T* dout, int M, int N, int64_t ld, float* partial, size_t partial_floats,
                     hipStream_t s);
// Fused softmax cross-entropy: losses[i] = logsumexp(z_i) - z_i[y_i]; z_i is
// overwritten by (softmax(z_i) - onehot(y_i)) * dscale; padding columns V..ldz-1 zeroed.
template <class T>
hipError_t crossentropy_fused(T* logits, float* losses, const int32_t* targets, int N, int V, int64_t ldz,
                              float dscale, hipStream_t s, uint8_t* q = nullptr, int64_t ldq = 0,
                              uint8_t* sc = nullptr);
hipError_t mean_loss(float* loss, const float* losses, int N, hipStream_t s);
hipError_t scaled_accumulate(float* dst, const float* src, float scale, bool first, hipStream_t s);
// dwte[tok] += dx rows (deterministic), dwpe[t] = sum_b dx[b, t] for t < T, 0 for T <= t < P.
// first / count: int [V] scratch, INT_MAX / 0 on entry (token_census_reset) and on return.
// AdamW of a parameter range inside another kernel (p null: no update).
struct AdamwRows {
    float* p;
    float* m;
    float* v;
    bf16* p16;
    float lr, b1, b2, eps, wd, c1, c2;
};
// token_census: first position and count of every token id of tok [BT] (the census
// must hold its idle state: first = INT_MAX, count = 0; encoder_backward restores it).
hipError_t token_census(int* first, int* count, const int32_t* tok, int BT, hipStream_t s);
// Needs the census of tok.  With opt.p set, each present token's row of wte gets its
// AdamW update right after its gradient is complete.
template <class T>
hipError_t encoder_backward(float* dwte, float* dwpe, const T* dx, const int32_t* tok, int B, int T_, int P, int C,
                            int* first, int* count, hipStream_t s, bool wpe_used = true,
                            const AdamwRows& opt = AdamwRows{});
// AdamW over the rows r < rows (C values each) of a matrix whose count[r] == 0.
hipError_t adamw_rows_absent(const AdamwRows& o, const float* g, const int* count, int rows, int C, hipStream_t s);
hipError_t token_census_reset(int* first, int* count, int V, hipStream_t s);
hipError_t adamw(float* p, const float* g, float* m, float* v, bf16* p16, int64_t n, float lr, float b1, float b2,
                 float eps, float wd, float c1, float c2, hipStream_t s);
hipError_t cast_bf16(bf16* out, const float* in, int64_t n, hipStream_t s);
// out[i] = sum over k < splits of ws[k * stride + i], i < n (fixed order).
hipError_t splitk_reduce(float* out, const float* ws, int splits, int64_t n, int64_t stride, hipStream_t s);
// C (bf16 [M, N], row stride ldc) = bias + sum of `splits` dense fp32 M x N partials.
// MX FP8 ("1000 行 C 代码完成 GPT-2 训练的 LLM.c": precision below 16 bits).  E4M3
// codes with one power-of-two scale per 32 values along k.
// mx_quantize: x bf16 [R, K] (row stride ldx elements, K % 8 == 0) -> q [R, Kp] codes
// (row stride ldq bytes, Kp = K rounded up to 128, zero codes past K) and the scales
// sc [Kp / 128][R][4] (see GemmArgs).  Scale of a block: the smallest 2^e with
// amax <= 448 * 2^e (e in [-127, 127], all-zero blocks -127); codes: x / 2^e rounded
// to nearest even.
// MX codes of a weight W [R, K] (bf16): blocks along K into (q, sq) and, with qt, blocks
// along R -- the rows of W^T, rows past R as zero -- into (qt, sqt); layouts as
// mx_quantize's.
// With batch > 1, `batch` equally shaped weights at the given element / byte strides
// (one per layer) in one launch.
struct MxWeightStrides {
    int64_t w = 0, q = 0, sq = 0, qt = 0, sqt = 0;
};
hipError_t mx_weight_codes(const bf16* w, int64_t ldw, int R, int K, uint8_t* q, int64_t ldq, uint8_t* sq,
                           uint8_t* qt, int64_t ldqt, uint8_t* sqt, hipStream_t s, int batch = 1,
                           const MxWeightStrides& bs = MxWeightStrides{});
hipError_t mx_quantize(const bf16* x, int64_t ldx, int R, int K, uint8_t* q, int64_t ldq, uint8_t* sc,
                       hipStream_t s);
// C = A B^T (+ the epilogue) for MX operands: A codes [M, K] (lda bytes), B codes
// [N, K] (ldb bytes), K a multiple of 128 (zero-padded), lda / ldb multiples of 16;
// scales a.sa / a.sb; output bf16 with EPI_BIAS, EPI_BIAS_RES or EPI_BIAS_GELU.
hipError_t gemm_mx(const GemmArgs& a, int epi, hipStream_t s);

// Rotary position embedding: tab [P][hs / 2] (cos, sin) of m base^(-2i / hs), built in
// float64; rope_apply turns, in place, the pairs of the first ncols columns (whole
// heads of size hs) of rows x[r] (row stride ld) for position pos0 + r % period
// (inverse: turns back).
hipError_t rope_table(float2* tab, int P, int hs, double base, hipStream_t s);
template <class T>
hipError_t rope_apply(T* x, int64_t ld, int rows, int ncols, int hs, int period, int pos0, const float2* tab,
                      bool inverse, hipStream_t s);

// SwiGLU MLP of the Llama-style block: gu [N, 2H] holds (gate, up) of hidden unit j in
// columns 2j, 2j+1; forward h [N, H] = silu(g) * u; backward dgu = (dh u silu'(g),
// dh silu(g)) (overwrites).  H % 8 == 0.
template <class T>
hipError_t swiglu_forward(T* h, const T* gu, int N, int H, hipStream_t s);
template <class T>
hipError_t swiglu_backward(T* dgu, const T* dh, const T* gu, int N, int H, hipStream_t s);

hipError_t splitk_reduce_bf16(bf16* C, int64_t ldc, const float* ws, int splits, int M, int N, const float* bias,
                              hipStream_t s);

// ---------------------------------------------------------------- attention
// qkv [B*T, 3C] (q | k | v, head h at columns h*hs), out [B*T, C], lse fp32 [B, NH, T].
// q, sc (bf16 only): MX FP8 codes [B*T, ldq] and scales [C / 128][B*T][4] of out, written
// by the kernel when it can (head size 64, C % 128 == 0); *coded tells whether it did.
template <class T>
hipError_t attention_forward(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s,
                             uint8_t* q = nullptr, int64_t ldq = 0, uint8_t* sc = nullptr, bool* coded = nullptr);
// dqkv [B*T, 3C] (overwrite) from dout [B*T, C]; `dsum` fp32 [B, NH, T, 2] scratch.
template <class T>
hipError_t attention_backward(T* dqkv, float* dsum, const T* dout, const T* out, const T* qkv, const float* lse,
                              int B, int T_, int C, int NH, hipStream_t s);

// MFMA kernels for bf16 operands with head size 64 (used by the two above when they apply).
hipError_t attention_forward_mfma64(bf16* out, float* lse, const bf16* qkv, int B, int T_, int C, int NH,
                                    hipStream_t s, uint8_t* q = nullptr, int64_t ldq = 0, uint8_t* sc = nullptr);
hipError_t attention_backward_mfma64(bf16* dqkv, float* dsum, const bf16* dout, const bf16* out, const bf16* qkv,
                                     const float* lse, int B, int T_, int C, int NH, hipStream_t s);

// ---------------------------------------------------------------- generation (bf16)
// Skinny product for the rows of a decode step: C[m, n] = epilogue(sum_k x[m, k] W[n, k]),
// M <= 16, W [N, K] row-major; epilogues EPI_BIAS, EPI_BIAS_RES (+ R[m, n], row stride
// ldr), EPI_BIAS_GELU (C = pre-activation if non-null, C2 = gelu, both row stride ldc)
// and EPI_F32 (fp32 C = acc + bias).  K, ldx, ldw multiples of 8 (and with ln_w, the
// gains / shifts 16-byte aligned).
struct SkinnyArgs {
    const bf16* x;
    int64_t ldx;
    const bf16* W;
    int64_t ldw;
    void* C;
    int64_t ldc;
    bf16* C2;
    const bf16* R;
    int64_t ldr;
    const float* bias;
    // non-null: x is replaced by LayerNorm(x) with these fp32 gains / shifts [K]
    const float* ln_w;
    const float* ln_b;
    int M, N, K;
};
hipError_t skinny_gemm(const SkinnyArgs& a, int epi, hipStream_t s);
// y [batch, C] = attention of the query in cache row len-1 of each sequence over cache
// rows 0 .. len-1 (q | k | v rows of 3C, sequence b at cache + b * bstride); head size 64.
hipError_t attention_decode(bf16* y, const bf16* cache, int batch, int len, int C, int NH, int64_t bstride,
                            hipStream_t s);
// out fp32 [R, V] = rows (r * row_stride + row_offset) of bf16 logits with row stride ldl.
hipError_t logits_rows(float* out, const bf16* logits, int R, int V, int64_t ldl, int row_stride, int row_offset,
                       hipStream_t s);

}  // namespace gpt2
