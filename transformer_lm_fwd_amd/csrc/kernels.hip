// Memory-bound kernels of the GPT-2 training step (gfx950, wave64):
// embedding gather / scatter, LayerNorm forward / backward, bias gradients,
// fused softmax cross-entropy, AdamW, and small reductions.
#include "kernels.h"
#include "mx_quant.h"

namespace gpt2 {

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// ============================================================================ encoder
// "GPT-2 from scratch with torch", token/position embedding: x[b, t] = wte[tok[b, t]] + wpe[t].
// Reads the fp32 master tables and rounds once to the activation type.
template <class T>
__global__ __launch_bounds__(256) void encoder_forward_kernel(T* out, const int32_t* tok, const float* wte,
                                                              const float* wpe, int BT, int T_, int C, int pos0) {
    const int c4 = C / 4;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)BT * c4) return;
    int row = (int)(i / c4), c = (int)(i % c4) * 4;
    int t = pos0 + row % T_;
    float4 a = *(const float4*)(wte + (int64_t)tok[row] * C + c);
    // no wpe: positions enter through the rotary embedding of the queries and keys
    float4 p = wpe ? *(const float4*)(wpe + (int64_t)t * C + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    T* o = out + (int64_t)row * C + c;
    o[0] = from_f32<T>(a.x + p.x);
    o[1] = from_f32<T>(a.y + p.y);
    o[2] = from_f32<T>(a.z + p.z);
    o[3] = from_f32<T>(a.w + p.w);
}

template <class T>
hipError_t encoder_forward(T* out, const int32_t* tok, const float* wte, const float* wpe, int BT, int T_, int C,
                           hipStream_t s, int pos0) {
    ProfScope prof(s, "encoder_fwd", 0, (double)BT * C * (8 + sizeof(T)));
    hipLaunchKernelGGL(encoder_forward_kernel<T>, dim3(cdiv((int64_t)BT * (C / 4), 256)), dim3(256), 0, s, out, tok,
                       wte, wpe, BT, T_, C, pos0);
    return hipGetLastError();
}

// ============================================================================ LayerNorm forward
// "GPT-2 from scratch with torch", Transformer block (LayerNorm, eps 1e-5): per row
// mean and biased variance over C; y = (x - mean) * rstd * w + b.  One wave per row;
// the row stays in registers between the two statistics passes.
// MXO: also writes the MX FP8 codes and block scales of the (bf16-rounded) output,
// q [N, Kp] (row stride ldq bytes), sc [Kp / 128][N][4], for a following MX product;
// lane l's 8 values are chunk 64 ch + l, so 4 lanes hold a 32-block and 16 a stage.
// rms: RMSNorm (Llama-style block) - the mean is taken as 0 (the statistics hold
// mean 0 and 1 / sqrt(mean(x^2) + eps)); b may be null (no shift).
// Each wave takes RPW consecutive rows; the next row's loads go out before the current
// row is reduced, and the gains / shifts are loaded once per wave.
// MXO: also writes the MX FP8 codes and block scales of the (bf16-rounded) output,
// q [N, Kp] (row stride ldq bytes), sc [Kp / 128][N][4], for a following MX product;
// lane l's 8 values are chunk 64 ch + l, so 4 lanes hold a 32-block and 16 a stage.
#ifndef LNF_RPW
#define LNF_RPW 1
#endif
template <class T, int MAXCH, bool MXO = false, int RPW = LNF_RPW>
__global__ __launch_bounds__(256) void layernorm_forward_kernel(T* out, float* stats, const T* inp, const float* w,
                                                                const float* b, int N, int C, uint8_t* q = nullptr,
                                                                int64_t ldq = 0, uint8_t* sc = nullptr,
                                                                bool rms = false) {
    constexpr int KV = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW;
    if (row0 >= N) return;
    float wv[MAXCH][KV], bv[MAXCH][KV];
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
        const int c = (ch * 64 + lane) * KV;
#pragma unroll
        for (int e = 0; e < KV; ++e) wv[ch][e] = bv[ch][e] = 0.f;
        if (c < C) {
#pragma unroll
            for (int e = 0; e < KV; e += 4) {  // C % 8 == 0: 16-byte aligned fp32 gains and shifts
                *(float4*)&wv[ch][e] = *(const float4*)(w + c + e);
                if (b) *(float4*)&bv[ch][e] = *(const float4*)(b + c + e);
            }
        }
    }
    u32x4 raw[MAXCH];
    auto issue = [&](int row) {
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            const int c = (ch * 64 + lane) * KV;
            raw[ch] = (row < N && c < C) ? ld16(inp + (int64_t)row * C + c) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    issue(row0);
#pragma unroll 1
    for (int i = 0; i < RPW; ++i) {
        const int row = row0 + i;
        if (row >= N) break;  // wave-uniform
        float v[MAXCH][KV];
        float sum = 0.f;
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            unpack16<T>(raw[ch], v[ch]);  // zeros past C
#pragma unroll
            for (int e = 0; e < KV; ++e) sum += v[ch][e];
        }
        if (i + 1 < RPW) issue(row + 1);
        const float mean = rms ? 0.f : wave_sum(sum) / C;
        float sq = 0.f;
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            const int c = (ch * 64 + lane) * KV;
            if (c < C) {
#pragma unroll
                for (int e = 0; e < KV; ++e) {
                    const float d = v[ch][e] - mean;
                    sq += d * d;
                }
            }
        }
        const float rstd = 1.0f / sqrtf(wave_sum(sq) / C + 1e-5f);
        T* y = out + (int64_t)row * C;
        if constexpr (MXO) {
            static_assert(KV == 8, "MX output from bf16 rows");
            const int Kp = (C + 127) / 128 * 128;
#pragma unroll
            for (int ch = 0; ch < MAXCH; ++ch) {
                const int c = (ch * 64 + lane) * KV;
                float o[KV];
#pragma unroll
                for (int e = 0; e < KV; ++e) o[e] = 0.f;
                if (c < C) {
#pragma unroll
                    for (int e = 0; e < KV; ++e) o[e] = (v[ch][e] - mean) * rstd * wv[ch][e] + bv[ch][e];
                    round_bf16_8(o);
                    st16(y + c, pack16<T>(o));
                }
                uint32_t cw[2];
                const uint32_t word = mx_stage_word(mx_quant8(o, cw));
                if (c < Kp) {
                    *(uint2*)(q + (int64_t)row * ldq + c) = make_uint2(cw[0], cw[1]);
                    if ((lane & 15) == 0) *(uint32_t*)(sc + ((int64_t)(c / 128) * N + row) * 4) = word;
                }
            }
        } else {
#pragma unroll
            for (int ch = 0; ch < MAXCH; ++ch) {
                const int c = (ch * 64 + lane) * KV;
                if (c < C) {
                    float o[KV];
#pragma unroll
                    for (int e = 0; e < KV; ++e) o[e] = (v[ch][e] - mean) * rstd * wv[ch][e] + bv[ch][e];
                    st16(y + c, pack16<T>(o));
                }
            }
        }
        if (lane == 0) {
            stats[2 * row] = mean;
            stats[2 * row + 1] = rstd;
        }
    }
}

template <class T>
hipError_t layernorm_forward(T* out, float* stats, const T* inp, const float* w, const float* b, int N, int C,
                             hipStream_t s, uint8_t* mxq, int64_t ldq, uint8_t* mxs, bool rms) {
    constexpr int KV = Vec16<T>::N;
    int ch = cdiv(C, 64 * KV);
    dim3 grid(cdiv(N, 4 * LNF_RPW)), block(256);
    if constexpr (sizeof(T) == 2) {
        if (mxq) {
            if (!mxs || ldq < (C + 127) / 128 * 128 || ldq % 16) return hipErrorInvalidValue;
            ProfScope prof(s, "layernorm_fwd_mx", 0, (double)N * C * 2 * sizeof(T) + 8.0 * N + N * C * (1 + 1 / 32.));
            if (ch <= 1)
                hipLaunchKernelGGL((layernorm_forward_kernel<T, 1, true>), grid, block, 0, s, out, stats, inp, w, b, N, C, mxq, ldq, mxs, rms);
            else if (ch <= 2)
                hipLaunchKernelGGL((layernorm_forward_kernel<T, 2, true>), grid, block, 0, s, out, stats, inp, w, b, N, C, mxq, ldq, mxs, rms);
            else if (ch <= 4)
                hipLaunchKernelGGL((layernorm_forward_kernel<T, 4, true>), grid, block, 0, s, out, stats, inp, w, b, N, C, mxq, ldq, mxs, rms);
            else return hipErrorInvalidValue;
            return hipGetLastError();
        }
    }
    if (mxq) return hipErrorInvalidValue;
    ProfScope prof(s, "layernorm_fwd", 0, (double)N * C * 2 * sizeof(T) + 8.0 * N);
    if (ch <= 1) hipLaunchKernelGGL((layernorm_forward_kernel<T, 1>), grid, block, 0, s, out, stats, inp, w, b, N, C, nullptr, 0, nullptr, rms);
    else if (ch <= 2) hipLaunchKernelGGL((layernorm_forward_kernel<T, 2>), grid, block, 0, s, out, stats, inp, w, b, N, C, nullptr, 0, nullptr, rms);
    else if (ch <= 4) hipLaunchKernelGGL((layernorm_forward_kernel<T, 4>), grid, block, 0, s, out, stats, inp, w, b, N, C, nullptr, 0, nullptr, rms);
    else if (ch <= 8) hipLaunchKernelGGL((layernorm_forward_kernel<T, 8>), grid, block, 0, s, out, stats, inp, w, b, N, C, nullptr, 0, nullptr, rms);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// ============================================================================ LayerNorm backward
// With xhat = (x - mean) * rstd and dxhat = dy * w:
//   dx = rstd * (dxhat - mean_c(dxhat) - xhat * mean_c(dxhat * xhat))   (written or added into dres)
//   dw = sum_rows dy * xhat,  db = sum_rows dy                          (column sums, below)
// dx: one wave per row, the row's dy and x held in registers.
// rms: RMSNorm's backward - without the mean_c(dxhat) term (the statistics' mean is 0).
template <class T, int MAXCH>
__global__ __launch_bounds__(256) void layernorm_backward_dx_kernel(T* dres, const T* dres_in, const T* dout,
                                                                    const T* inp, const float* stats, const float* w,
                                                                    int N, int C, bool rms) {
    constexpr int KV = Vec16<T>::N;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= N) return;
    const float mean = stats[2 * row], rstd = stats[2 * row + 1];
    const T* dy = dout + (int64_t)row * C;
    const T* x = inp + (int64_t)row * C;
    float g[MAXCH][KV], xh[MAXCH][KV];
    float s1 = 0.f, s2 = 0.f;
    const T* dxi = dres_in ? dres_in + (int64_t)row * C : nullptr;
    u32x4 prev_raw[MAXCH];  // the residual gradient to add, requested before the reductions
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
        const int c = (ch * 64 + lane) * KV;
        prev_raw[ch] = (dxi && c < C) ? ld16(dxi + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
        const int c = (ch * 64 + lane) * KV;
        if (c < C) {
            float wv[KV];
            unpack16<T>(ld16(dy + c), g[ch]);
            unpack16<T>(ld16(x + c), xh[ch]);
            unpack16<float>(ld16(w + c), wv);
            if constexpr (KV == 8) unpack16<float>(ld16(w + c + 4), wv + 4);
#pragma unroll
            for (int e = 0; e < KV; ++e) {
                xh[ch][e] = (xh[ch][e] - mean) * rstd;
                g[ch][e] *= wv[e];  // dxhat
                s1 += g[ch][e];
                s2 += g[ch][e] * xh[ch][e];
            }
        }
    }
    s1 = rms ? 0.f : wave_sum(s1) / C;
    s2 = wave_sum(s2) / C;
    T* dx = dres + (int64_t)row * C;
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
        const int c = (ch * 64 + lane) * KV;
        if (c < C) {
            float prev[KV], o[KV];
            unpack16<T>(prev_raw[ch], prev);
#pragma unroll
            for (int e = 0; e < KV; ++e) o[e] = rstd * (g[ch][e] - s1 - xh[ch][e] * s2) + prev[e];
            st16(dx + c, pack16<T>(o));
        }
    }
}

// Column sums over M rows (deterministic, two stages).
// Stage 1: block (x: 64*KV columns, y: a chunk of rows); each lane owns KV columns
// (one 16-byte load per row), the four waves take interleaved rows, and the block's
// sums go to partial[blockIdx.y][...].  With LN, xhat is rebuilt from (mean, rstd):
// partial row = [sum dy * xhat (N) | sum dy (N)]; without, [sum dy (N)].
template <class T, bool LN>
__global__ __launch_bounds__(256) void colsum_stage1_kernel(float* partial, const T* dy, const T* x,
                                                            const float* stats, int M, int N, int64_t ld,
                                                            int rows_per) {
    constexpr int KV = Vec16<T>::N;
    constexpr int NS = LN ? 2 : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int c = (blockIdx.x * 64 + lane) * KV;
    const int r0 = blockIdx.y * rows_per, r1 = min(M, r0 + rows_per);
    float sb[KV], sw[KV];
#pragma unroll
    for (int e = 0; e < KV; ++e) sb[e] = sw[e] = 0.f;
    if (c < N) {
        for (int r = r0 + wave; r < r1; r += 4) {
            float gv[KV];
            unpack16<T>(ld16(dy + (int64_t)r * ld + c), gv);
            if constexpr (LN) {
                float xv[KV];
                unpack16<T>(ld16(x + (int64_t)r * ld + c), xv);
                const float mean = stats[2 * r], rstd = stats[2 * r + 1];
#pragma unroll
                for (int e = 0; e < KV; ++e) sw[e] += gv[e] * ((xv[e] - mean) * rstd);
            }
#pragma unroll
            for (int e = 0; e < KV; ++e) sb[e] += gv[e];
        }
    }
    __shared__ float red[4][NS][64 * KV];
#pragma unroll
    for (int e = 0; e < KV; ++e) {
        red[wave][0][lane * KV + e] = sb[e];
        if constexpr (LN) red[wave][NS - 1][lane * KV + e] = sw[e];
    }
    __syncthreads();
    const int W = NS * N;
    float* out = partial + (int64_t)blockIdx.y * W;
    for (int i = threadIdx.x; i < NS * 64 * KV; i += 256) {
        const int sidx = i / (64 * KV), j = i % (64 * KV);
        const int col = blockIdx.x * 64 * KV + j;
        if (col < N) {
            float v = (red[0][sidx][j] + red[1][sidx][j]) + (red[2][sidx][j] + red[3][sidx][j]);
            // LN: sums of dy*xhat first (dw), then sums of dy (db)
            const int dst = LN ? (sidx == 1 ? col : N + col) : col;
            out[dst] = v;
        }
    }
}

// Stage 2: out[c] = sum over nb partial rows (fixed order).  A block takes 16
// columns; its 256 threads are 16 columns x 16 row lanes, lane k summing partial
// rows k, k+16, ...; the 16 lane sums are then added in order.
__global__ __launch_bounds__(256) void colsum_stage2_kernel(float* out0, float* out1, const float* partial, int nb,
                                                            int W, int split) {
    const int cl = threadIdx.x & 15, kl = threadIdx.x >> 4;
    const int c = blockIdx.x * 16 + cl;
    float acc = 0.f;
    if (c < W) {
#pragma unroll 16
        for (int k = kl; k < nb; k += 16) acc += partial[(int64_t)k * W + c];
    }
    __shared__ float red[16][16];
    red[kl][cl] = acc;
    __syncthreads();
    if (threadIdx.x < 16 && c < W) {
        float v = 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) v += red[k][cl];
        if (c < split) out0[c] = v;
        else if (out1) out1[c - split] = v;  // null: no shift parameter (RMSNorm)
    }
}

template <class T, bool LN>
static hipError_t colsum(float* out0, float* out1, const T* dy, const T* x, const float* stats, int M, int N,
                         int64_t ld, float* partial, size_t partial_floats, hipStream_t s, const char* name) {
    constexpr int KV = Vec16<T>::N;
    const int NS = LN ? 2 : 1;
    const int bx = cdiv(N, 64 * KV);
    int rb = 1;
    while (rb * bx < 1024 && rb < 256) rb *= 2;
    while ((size_t)rb * NS * N > partial_floats && rb > 1) rb /= 2;
    if ((size_t)rb * NS * N > partial_floats) return hipErrorInvalidValue;
    const int rows_per = cdiv(M, rb);
    rb = cdiv(M, rows_per);
    {
        ProfScope prof(s, name, 0, (double)M * N * sizeof(T) * (LN ? 2 : 1) + 4.0 * rb * NS * N);
        hipLaunchKernelGGL((colsum_stage1_kernel<T, LN>), dim3(bx, rb), dim3(256), 0, s, partial, dy, x, stats, M, N,
                           ld, rows_per);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ProfScope prof2(s, "colsum_stage2", 0, 4.0 * rb * NS * N + 4.0 * NS * N);
    hipLaunchKernelGGL(colsum_stage2_kernel, dim3(cdiv(NS * N, 16)), dim3(256), 0, s, out0, out1, partial, rb, NS * N,
                       N);
    return hipGetLastError();
}

template <class T>
hipError_t layernorm_backward_dx(T* dres, const T* dres_in, const T* dout, const T* inp, const float* stats,
                                 const float* w, int N, int C, hipStream_t s, bool rms) {
    constexpr int KV = Vec16<T>::N;
    const int ch = cdiv(C, 64 * KV);
    const dim3 grid(cdiv(N, 4)), block(256);
    ProfScope prof(s, "layernorm_bwd_dx", 0, (double)N * C * sizeof(T) * (dres_in ? 4 : 3) + 8.0 * N);
    if (ch <= 1) hipLaunchKernelGGL((layernorm_backward_dx_kernel<T, 1>), grid, block, 0, s, dres, dres_in, dout, inp, stats, w, N, C, rms);
    else if (ch <= 2) hipLaunchKernelGGL((layernorm_backward_dx_kernel<T, 2>), grid, block, 0, s, dres, dres_in, dout, inp, stats, w, N, C, rms);
    else if (ch <= 4) hipLaunchKernelGGL((layernorm_backward_dx_kernel<T, 4>), grid, block, 0, s, dres, dres_in, dout, inp, stats, w, N, C, rms);
    else if (ch <= 8) hipLaunchKernelGGL((layernorm_backward_dx_kernel<T, 8>), grid, block, 0, s, dres, dres_in, dout, inp, stats, w, N, C, rms);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <class T>
hipError_t layernorm_param_grads(float* dw, float* db, const T* dout, const T* inp, const float* stats, int N, int C,
                                 float* partial, size_t partial_floats, hipStream_t s) {
    return colsum<T, true>(dw, db, dout, inp, stats, N, C, C, partial, partial_floats, s, "layernorm_bwd_dwdb");
}

// dx and the parameter-gradient partials in one pass: each of the 8 waves takes RPW
// rows (row = (block * RPW + i) * 8 + wave), computing dx as above while it adds
// dy * xhat and dy into per-lane column sums; the loads of row i + 1 are issued
// before row i is reduced.  The block's eight wave sums (added in a fixed order)
// form partial row blockIdx.x = [sum dy * xhat (C) | sum dy (C)]; the second
// column-sum stage adds the partial rows.
template <class T, int MAXCH, int RPW>
__global__ __launch_bounds__(512) void layernorm_backward_fused_kernel(T* dres, float* partial, const T* dres_in,
                                                                       const T* dout, const T* inp,
                                                                       const float* stats, const float* w, int N,
                                                                       int C, bool rms, uint8_t* q, int64_t ldq,
                                                                       uint8_t* sc) {
    constexpr int KV = Vec16<T>::N;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float wv[MAXCH][KV], aw[MAXCH][KV], ab[MAXCH][KV];
#pragma unroll
    for (int ch = 0; ch < MAXCH; ++ch) {
        const int c = (ch * 64 + lane) * KV;
#pragma unroll
        for (int e = 0; e < KV; ++e) {
            aw[ch][e] = ab[ch][e] = 0.f;
            wv[ch][e] = 0.f;
        }
        if (c < C) {
#pragma unroll
            for (int e = 0; e < KV; e += 4) *(float4*)&wv[ch][e] = *(const float4*)(w + c + e);
        }
    }
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    u32x4 rg[MAXCH], rx[MAXCH], rp[MAXCH];  // raw dy, x, residual gradient of the current row
    auto issue = [&](int row) {
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            const int c = (ch * 64 + lane) * KV;
            const bool ok = row < N && c < C;
            rg[ch] = ok ? ld16(dout + (int64_t)row * C + c) : z4;
            rx[ch] = ok ? ld16(inp + (int64_t)row * C + c) : z4;
            rp[ch] = (ok && dres_in) ? ld16(dres_in + (int64_t)row * C + c) : z4;
        }
    };
    const int row0 = blockIdx.x * RPW * 8 + wave;
    issue(row0);
#pragma unroll 1
    for (int i = 0; i < RPW; ++i) {
        const int row = row0 + 8 * i;
        float g[MAXCH][KV], xh[MAXCH][KV], prev[MAXCH][KV];
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            unpack16<T>(rg[ch], g[ch]);
            unpack16<T>(rx[ch], xh[ch]);
            unpack16<T>(rp[ch], prev[ch]);
        }
        if (i + 1 < RPW) issue(row + 8);
        if (row >= N) break;  // wave-uniform; later rows are past the end too
        const float mean = stats[2 * row], rstd = stats[2 * row + 1];
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch)
#pragma unroll
            for (int e = 0; e < KV; ++e) {  // lanes past C hold zeros and add nothing
                xh[ch][e] = (xh[ch][e] - mean) * rstd;
                aw[ch][e] += g[ch][e] * xh[ch][e];
                ab[ch][e] += g[ch][e];
                g[ch][e] *= wv[ch][e];  // dxhat
                s1 += g[ch][e];
                s2 += g[ch][e] * xh[ch][e];
            }
        s1 = rms ? 0.f : wave_sum(s1) / C;
        s2 = wave_sum(s2) / C;
        T* dx = dres + (int64_t)row * C;
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            const int c = (ch * 64 + lane) * KV;
            float o[KV];
#pragma unroll
            for (int e = 0; e < KV; ++e) o[e] = c < C ? rstd * (g[ch][e] - s1 - xh[ch][e] * s2) + prev[ch][e] : 0.f;
            if (c < C) st16(dx + c, pack16<T>(o));
            if constexpr (sizeof(T) == 2) {
                // MX codes of the stored row (the next input-gradient product's upstream
                // gradient): lanes 4j .. 4j+3 a 32-block, 16j .. 16j+15 a 128-stage; the
                // columns past C quantize as zeros
                if (q) {  // block-uniform
                    round_bf16_8(o);
                    uint32_t cw[2];
                    const uint32_t word = mx_stage_word(mx_quant8(o, cw));
                    if (c < ldq) {
                        *(uint2*)(q + (int64_t)row * ldq + c) = make_uint2(cw[0], cw[1]);
                        if ((lane & 15) == 0) *(uint32_t*)(sc + ((int64_t)(c / 128) * N + row) * 4) = word;
                    }
                }
            }
        }
    }
    // The eight wave sums go through 16 KB of LDS, one (sum, chunk) pair at a time, so
    // that a block fits beside a 144 KB matrix-product block of the other stream.
    __shared__ float red[8][64 * KV];
    float* out = partial + (int64_t)blockIdx.x * 2 * C;
#pragma unroll
    for (int sidx = 0; sidx < 2; ++sidx)
#pragma unroll
        for (int ch = 0; ch < MAXCH; ++ch) {
            if (ch * 64 * KV >= C) break;  // block-uniform
#pragma unroll
            for (int e = 0; e < KV; ++e) red[wave][lane * KV + e] = sidx == 0 ? aw[ch][e] : ab[ch][e];
            __syncthreads();
            for (int i = threadIdx.x; i < 64 * KV; i += 512) {
                const int c = ch * 64 * KV + i;
                if (c < C)
                    out[sidx * C + c] = ((red[0][i] + red[1][i]) + (red[2][i] + red[3][i])) +
                                        ((red[4][i] + red[5][i]) + (red[6][i] + red[7][i]));
            }
            __syncthreads();
        }
}

template <class T>
hipError_t layernorm_backward(T* dres, const T* dres_in, float* dw, float* db, const T* dout, const T* inp,
                              const float* stats, const float* w, int N, int C, float* partial, size_t partial_floats,
                              hipStream_t s, bool rms, uint8_t* q, int64_t ldq, uint8_t* sc) {
    constexpr int KV = Vec16<T>::N;
    if (q && (sizeof(T) != 2 || !sc || ldq % 128 || ldq < C)) return hipErrorInvalidValue;
    const int ch = cdiv(C, 64 * KV);
    // rows per wave: about 256 blocks for the step's 8192 rows, fewer rows for small inputs
    int rpw = 1;
    while (rpw < 4 && (int64_t)cdiv(N, 8 * rpw) > 256) rpw *= 2;
    while ((size_t)cdiv(N, 8 * rpw) * 2 * C > partial_floats && rpw < 64) rpw *= 2;
    const int nb = cdiv(N, 8 * rpw);
    if ((size_t)nb * 2 * C > partial_floats || ch > 2 || (rpw != 1 && rpw != 2 && rpw != 4)) {
        hipError_t e = layernorm_backward_dx<T>(dres, dres_in, dout, inp, stats, w, N, C, s, rms);
        if (e != hipSuccess) return e;
        if (q) {  // (codes of the written rows by the standalone quantizer)
            if constexpr (sizeof(T) == 2) e = mx_quantize((const bf16*)dres, C, N, C, q, ldq, sc, s);
            if (e != hipSuccess) return e;
        }
        return layernorm_param_grads<T>(dw, db, dout, inp, stats, N, C, partial, partial_floats, s);
    }
    {
        ProfScope prof(s, "layernorm_bwd", 0, (double)N * C * sizeof(T) * (dres_in ? 4 : 3) + 8.0 * N + 8.0 * nb * C);
#define LNB_LAUNCH(MC, R)                                                                                             \
    hipLaunchKernelGGL((layernorm_backward_fused_kernel<T, MC, R>), dim3(nb), dim3(512), 0, s, dres, partial, dres_in, \
                       dout, inp, stats, w, N, C, rms, q, ldq, sc)
#define LNB_RPW(MC)                            \
    if (rpw == 1) LNB_LAUNCH(MC, 1);           \
    else if (rpw == 2) LNB_LAUNCH(MC, 2);      \
    else LNB_LAUNCH(MC, 4);
        if (ch <= 1) { LNB_RPW(1) }
        else { LNB_RPW(2) }
#undef LNB_RPW
#undef LNB_LAUNCH
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ProfScope prof2(s, "colsum_stage2", 0, 4.0 * nb * 2 * C + 8.0 * C);
    hipLaunchKernelGGL(colsum_stage2_kernel, dim3(cdiv(2 * C, 16)), dim3(256), 0, s, dw, db, partial, nb, 2 * C, C);
    return hipGetLastError();
}

// ============================================================================ bias gradients
// dbias[n] = sum_m dout[m, n] (overwrite).
template <class T>
hipError_t bias_grad(float* dbias, const T* dout, int M, int N, int64_t ld, float* partial, size_t partial_floats,
                     hipStream_t s) {
    return colsum<T, false>(dbias, dbias, dout, (const T*)nullptr, nullptr, M, N, ld, partial, partial_floats, s,
                            "bias_grad");
}

// ============================================================================ softmax cross-entropy
// "从头搭建GPT(Andrej Karpathy) 笔记", 计算loss: loss_i = logsumexp(z_i) - z_i[y_i]; the mean
// over the B*T rows is the training loss, so d loss / d z_i = (softmax(z_i) - onehot(y_i)) / (B*T).
// One block per row: an online (max, sum) pass, then the gradient overwrites z_i in place.
__device__ __forceinline__ void online_merge(float& m, float& s, float m2, float s2) {
    float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    s = s * __expf(m - mn) + s2 * __expf(m2 - mn);
    m = mn;
}

// The first REG 16-byte vectors of each thread's share of the row stay in registers
// between the two passes, so the logits are read from memory once (rows up to
// REG * 1024 vectors; longer rows re-read the rest).  Each thread first takes the
// maximum of its values, then sums 2^((z - m) log2 e) with one v_exp_f32 per value
// (log2 e folded into a multiply-add); the block merges the (max, sum) pairs.  The
// gradient pass spends one more exponential per value, with 1/(B*T) folded into the
// exponent's offset; the -1/(B*T) of the target column is added by the one thread
// whose vector holds it.
template <class T>
__global__ __launch_bounds__(1024) void crossentropy_kernel(T* logits, float* losses, const int32_t* targets, int V,
                                                            int64_t ldz, float dscale, uint8_t* q, int64_t ldq,
                                                            uint8_t* sc, int nrows) {
    constexpr int KV = Vec16<T>::N;
    constexpr int REG = 64 / KV;  // 64 values per thread: V up to 65536
    constexpr float L2E = 1.4426950408889634f;
    const int row = blockIdx.x;
    T* z = logits + (int64_t)row * ldz;
    const int nvec = V / KV;  // full 16-byte vectors inside [0, V)
    const int y = targets[row];
    const float zy = to_f32(z[y]);
    u32x4 keep[REG];
#pragma unroll
    for (int r = 0; r < REG; ++r) {
        const int i = threadIdx.x + r * 1024;
        if (i < nvec) keep[r] = ld16(z + i * KV);
    }
    // this thread's maximum
    float m = -INFINITY;
    auto vmax = [&](const u32x4& raw) {
        float v[KV];
        unpack16<T>(raw, v);
#pragma unroll
        for (int e = 0; e < KV; ++e) m = fmaxf(m, v[e]);
    };
#pragma unroll
    for (int r = 0; r < REG; ++r)
        if (threadIdx.x + r * 1024 < nvec) vmax(keep[r]);
    for (int i = threadIdx.x + REG * 1024; i < nvec; i += 1024) vmax(ld16(z + i * KV));
    for (int i = nvec * KV + threadIdx.x; i < V; i += 1024) m = fmaxf(m, to_f32(z[i]));
    // sum of 2^((z - m) log2 e) over this thread's values
    float s = 0.f;
    const float mo = m == -INFINITY ? 0.f : -m * L2E;
    auto vsum = [&](const u32x4& raw) {
        float v[KV];
        unpack16<T>(raw, v);
#pragma unroll
        for (int e = 0; e < KV; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], L2E, mo));
    };
#pragma unroll
    for (int r = 0; r < REG; ++r)
        if (threadIdx.x + r * 1024 < nvec) vsum(keep[r]);
    for (int i = threadIdx.x + REG * 1024; i < nvec; i += 1024) vsum(ld16(z + i * KV));
    for (int i = nvec * KV + threadIdx.x; i < V; i += 1024) s += __builtin_amdgcn_exp2f(__builtin_fmaf(to_f32(z[i]), L2E, mo));
    // block reduction of (m, s)
    __shared__ float sm[16], ss_[16];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        online_merge(m, s, m2, s2);
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { sm[wave] = m; ss_[wave] = s; }
    __syncthreads();
    m = sm[0]; s = ss_[0];
    for (int w2 = 1; w2 < 16; ++w2) online_merge(m, s, sm[w2], ss_[w2]);
    const float lse = m + __logf(s);
    if (threadIdx.x == 0) losses[row] = lse - zy;
    // dz = 2^(z log2 e - (lse log2 e - log2 dscale)) - [col == y] dscale
    const float go = -(lse * L2E - __log2f(dscale));
    auto grad = [&](const u32x4& raw, int i) {
        float v[KV];
        unpack16<T>(raw, v);
#pragma unroll
        for (int e = 0; e < KV; ++e) v[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[e], L2E, go));
        if ((unsigned)(y - i * KV) < (unsigned)KV) {
#pragma unroll
            for (int e = 0; e < KV; ++e)
                if (i * KV + e == y) v[e] -= dscale;
        }
        st16(z + i * KV, pack16<T>(v));
        if constexpr (sizeof(T) == 2) {
            // MX codes of a 128-value stage that lies wholly among the full vectors come
            // from the registers (its 16 lanes all run this branch); the rest are read
            // back below
            if (q && (i | 15) < nvec) {
                float t[KV];
#pragma unroll
                for (int e = 0; e < KV; ++e) t[e] = v[e];
                round_bf16_8(t);
                uint32_t cw[2];
                const uint32_t word = mx_stage_word(mx_quant8(t, cw));
                *(uint2*)(q + (int64_t)row * ldq + i * KV) = make_uint2(cw[0], cw[1]);
                if ((i & 15) == 0) *(uint32_t*)(sc + ((int64_t)(i / 16) * nrows + row) * 4) = word;
            }
        }
    };
#pragma unroll
    for (int r = 0; r < REG; ++r) {
        const int i = threadIdx.x + r * 1024;
        if (i < nvec) grad(keep[r], i);
    }
    for (int i = threadIdx.x + REG * 1024; i < nvec; i += 1024) grad(ld16(z + i * KV), i);
    for (int i = nvec * KV + threadIdx.x; i < (int)ldz; i += 1024) {
        float g = 0.f;
        if (i < V) g = __builtin_amdgcn_exp2f(__builtin_fmaf(to_f32(z[i]), L2E, go)) - (i == y ? dscale : 0.f);
        z[i] = from_f32<T>(g);
    }
    if constexpr (sizeof(T) == 2) {
        // MX codes of the stored gradient row (the tied lm_head's input-gradient product
        // takes them) from the stage that holds the row's end on: read back from L2 once
        // the block's stores are done, 4 threads per 32-block, 16 per 128-value stage;
        // columns past ldz are zero
        if (q) {  // block-uniform
            __syncthreads();
            const int nq = (int)(ldq / KV), nvs = nvec & ~15;
            for (int r = 0; r < (nq - nvs + 1023) / 1024; ++r) {  // every lane runs every round
                const int i = nvs + threadIdx.x + r * 1024;
                float v[KV];
                if (i < nq && (int64_t)(i + 1) * KV <= ldz) unpack16<T>(ld16(z + i * KV), v);
                else
#pragma unroll
                    for (int e = 0; e < KV; ++e) v[e] = 0.f;
                uint32_t cw[2];
                const uint32_t word = mx_stage_word(mx_quant8(v, cw));
                if (i < nq) {
                    *(uint2*)(q + (int64_t)row * ldq + i * KV) = make_uint2(cw[0], cw[1]);
                    if ((i & 15) == 0) *(uint32_t*)(sc + ((int64_t)(i / 16) * nrows + row) * 4) = word;
                }
            }
        }
    }
}

template <class T>
hipError_t crossentropy_fused(T* logits, float* losses, const int32_t* targets, int N, int V, int64_t ldz,
                              float dscale, hipStream_t s, uint8_t* q, int64_t ldq, uint8_t* sc) {
    if (q && (sizeof(T) != 2 || !sc || ldq % 128 || ldq < ldz || ldz % 8)) return hipErrorInvalidValue;
    ProfScope prof(s, q ? "crossentropy_mx" : "crossentropy", 0,
                   2.0 * N * ldz * sizeof(T) + 8.0 * N + (q ? N * ldq * (1 + 1 / 32.) : 0.0));
    hipLaunchKernelGGL(crossentropy_kernel<T>, dim3(N), dim3(1024), 0, s, logits, losses, targets, V, ldz, dscale, q,
                       ldq, sc, N);
    return hipGetLastError();
}

__global__ __launch_bounds__(1024) void mean_loss_kernel(float* loss, const float* losses, int N) {
    float acc = 0.f;
    for (int i = threadIdx.x; i < N; i += 1024) acc += losses[i];
    __shared__ float red[16];
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int w = 0; w < 16; ++w) t += red[w];
        loss[0] = t / N;
    }
}

// dst = src * scale (first) or dst += src * scale: a mean over a sequence of scalars
// enqueued one by one on a stream, added in that order.
__global__ void scaled_accumulate_kernel(float* dst, const float* src, float scale, int first) {
    if (threadIdx.x == 0) dst[0] = first ? src[0] * scale : dst[0] + src[0] * scale;
}

hipError_t scaled_accumulate(float* dst, const float* src, float scale, bool first, hipStream_t s) {
    ProfScope prof(s, "scaled_accumulate", 0, 12.0);
    hipLaunchKernelGGL(scaled_accumulate_kernel, dim3(1), dim3(64), 0, s, dst, src, scale, first ? 1 : 0);
    return hipGetLastError();
}

hipError_t mean_loss(float* loss, const float* losses, int N, hipStream_t s) {
    ProfScope prof(s, "mean_loss", 0, 4.0 * N);
    hipLaunchKernelGGL(mean_loss_kernel, dim3(1), dim3(1024), 0, s, loss, losses, N);
    return hipGetLastError();
}

// ============================================================================ encoder backward
// dwte[v] += sum of dx rows whose token is v.  The first position holding token v
// (its "leader") sums every matching row in increasing position order and is the
// only writer of dwte[v], so the result is deterministic without atomics on the
// sums.  A first pass records, per token, its first position (atomic minimum) and
// its number of occurrences (atomic add) -- both independent of thread order -- so a
// position learns whether it leads in O(1), and a leader of a token seen once adds
// its own row without scanning.  Repeated tokens are matched 256 positions at a time
// with wave ballots.  The leader re-arms first[v] / count[v] for the next call.
__global__ __launch_bounds__(256) void token_census_kernel(int* first, int* count, const int32_t* tok, int BT) {
    const int p = blockIdx.x * 256 + threadIdx.x;
    if (p >= BT) return;
    atomicMin(&first[tok[p]], p);
    atomicAdd(&count[tok[p]], 1);
}

// AdamW of one parameter ("1000 行 C 代码完成 GPT-2 训练的 LLM.c": the step ends with an
// Adam update).  Decoupled weight decay with bias correction (c1 = 1 - beta1^t,
// c2 = 1 - beta2^t): m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
// p -= lr (m/c1 / (sqrt(v/c2) + eps) + wd p)
// Every rounding is spelled out (fused multiply-adds, correctly rounded divisions and
// square root), so each kernel that applies the update - the whole-array pass, the
// absent-rows pass, the embedding scatter - produces the same bits whatever the
// compiler would otherwise contract.
__device__ __forceinline__ void adamw_one(float& p, float g, float& m, float& v, float lr, float b1, float b2,
                                          float eps, float wd, float c1, float c2) {
    m = __fmaf_rn(b1, m, (1.f - b1) * g);
    v = __fmaf_rn(b2, v, ((1.f - b2) * g) * g);
    const float mh = __fdiv_rn(m, c1), vh = __fdiv_rn(v, c2);
    const float u = __fmaf_rn(wd, p, __fdiv_rn(mh, __fsqrt_rn(vh) + eps));
    p = __fmaf_rn(-lr, u, p);
}

template <class T>
__global__ __launch_bounds__(256) void encoder_backward_wte_kernel(float* dwte, const T* dx, const int32_t* tok,
                                                                   int* first, int* count, int BT, int C,
                                                                   AdamwRows opt) {
    const int pos = blockIdx.x;
    const int v = tok[pos];
    if (first[v] != pos) return;  // block-uniform
    const int n = count[v];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    constexpr int MAXC = 8;  // columns per thread: C <= 2048
    float acc[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x + i * 256;
        acc[i] = c < C ? to_f32(dx[(int64_t)pos * C + c]) : 0.f;
    }
    if (n > 1) {
        __shared__ unsigned long long mask[4];
        int found = 1;
        for (int j0 = pos + 1; j0 < BT && found < n; j0 += 256) {
            const int j = j0 + threadIdx.x;
            const unsigned long long bal = __ballot((j < BT) && tok[j] == v);
            if (lane == 0) mask[wave] = bal;
            __syncthreads();
            for (int w = 0; w < 4; ++w) {
                unsigned long long mm = mask[w];
                while (mm) {
                    const int bit = __ffsll((long long)mm) - 1;
                    mm &= mm - 1;
                    const T* r = dx + (int64_t)(j0 + w * 64 + bit) * C;
#pragma unroll
                    for (int i = 0; i < MAXC; ++i) {
                        const int c = threadIdx.x + i * 256;
                        if (c < C) acc[i] += to_f32(r[c]);
                    }
                    ++found;
                }
            }
            __syncthreads();
        }
    }
    float* out = dwte + (int64_t)v * C;
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
        const int c = threadIdx.x + i * 256;
        if (c < C) {
            const float g = out[c] + acc[i];
            out[c] = g;
            if (opt.p) {  // the row's gradient is complete: its AdamW update
                const int64_t o = (int64_t)v * C + c;
                float pp = opt.p[o], mm = opt.m[o], vv = opt.v[o];
                adamw_one(pp, g, mm, vv, opt.lr, opt.b1, opt.b2, opt.eps, opt.wd, opt.c1, opt.c2);
                opt.p[o] = pp;
                opt.m[o] = mm;
                opt.v[o] = vv;
                if (opt.p16) opt.p16[o] = from_f32<bf16>(pp);
            }
        }
    }
    if (threadIdx.x == 0) {
        first[v] = 0x7fffffff;
        count[v] = 0;
    }
}

// AdamW over the rows of a matrix that no token of the batch touched (count == 0):
// their gradient is final before the embedding scatter.  Thread: 4 values of a row.
__global__ __launch_bounds__(256) void adamw_rows_absent_kernel(AdamwRows o, const float* g, const int* count, int rows,
                                                                int C) {
    const int c4 = C / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)rows * c4) return;
    const int r = (int)(i / c4);
    if (count[r] != 0) return;
    float4 pp = ((float4*)o.p)[i], mm = ((float4*)o.m)[i], vv = ((float4*)o.v)[i];
    const float4 gg = ((const float4*)g)[i];
    adamw_one(pp.x, gg.x, mm.x, vv.x, o.lr, o.b1, o.b2, o.eps, o.wd, o.c1, o.c2);
    adamw_one(pp.y, gg.y, mm.y, vv.y, o.lr, o.b1, o.b2, o.eps, o.wd, o.c1, o.c2);
    adamw_one(pp.z, gg.z, mm.z, vv.z, o.lr, o.b1, o.b2, o.eps, o.wd, o.c1, o.c2);
    adamw_one(pp.w, gg.w, mm.w, vv.w, o.lr, o.b1, o.b2, o.eps, o.wd, o.c1, o.c2);
    ((float4*)o.p)[i] = pp;
    ((float4*)o.m)[i] = mm;
    ((float4*)o.v)[i] = vv;
    if (o.p16) {
        uint2 h;
        h.x = pack2_bf16(pp.x, pp.y);
        h.y = pack2_bf16(pp.z, pp.w);
        ((uint2*)o.p16)[i] = h;
    }
}

hipError_t adamw_rows_absent(const AdamwRows& o, const float* g, const int* count, int rows, int C, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (C % 4) return hipErrorInvalidValue;
    ProfScope prof(s, "adamw_wte_absent", 0, (double)rows * C * 30.0);
    hipLaunchKernelGGL(adamw_rows_absent_kernel, dim3(cdiv((int64_t)rows * (C / 4), 256)), dim3(256), 0, s, o, g,
                       count, rows, C);
    return hipGetLastError();
}

hipError_t token_census(int* first, int* count, const int32_t* tok, int BT, hipStream_t s) {
    ProfScope prof(s, "token_census", 0, 4.0 * BT);
    hipLaunchKernelGGL(token_census_kernel, dim3(cdiv(BT, 256)), dim3(256), 0, s, first, count, tok, BT);
    return hipGetLastError();
}

__global__ void token_census_reset_kernel(int* first, int* count, int V) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < V) {
        first[i] = 0x7fffffff;
        count[i] = 0;
    }
}

hipError_t token_census_reset(int* first, int* count, int V, hipStream_t s) {
    hipLaunchKernelGGL(token_census_reset_kernel, dim3(cdiv(V, 256)), dim3(256), 0, s, first, count, V);
    return hipGetLastError();
}

// dwpe[t] = sum_b dx[b, t] for t < T; rows T..P-1 of dwpe get 0.
template <class T>
__global__ __launch_bounds__(256) void encoder_backward_wpe_kernel(float* dwpe, const T* dx, int B, int T_, int P,
                                                                   int C) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)P * C) return;
    int t = (int)(i / C), c = (int)(i % C);
    float acc = 0.f;
    if (t < T_)
        for (int b = 0; b < B; ++b) acc += to_f32(dx[((int64_t)b * T_ + t) * C + c]);
    dwpe[i] = acc;
}

template <class T>
hipError_t encoder_backward(float* dwte, float* dwpe, const T* dx, const int32_t* tok, int B, int T_, int P, int C,
                            int* first, int* count, hipStream_t s, bool wpe_used, const AdamwRows& opt) {
    if (C > 8 * 256) return hipErrorInvalidValue;
    hipError_t e;
    {
        ProfScope prof(s, "encoder_bwd_wte", 0, (double)B * T_ * C * (sizeof(T) + 8.0));
        hipLaunchKernelGGL(encoder_backward_wte_kernel<T>, dim3(B * T_), dim3(256), 0, s, dwte, dx, tok, first, count,
                           B * T_, C, opt);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    ProfScope prof2(s, "encoder_bwd_wpe", 0, (double)B * T_ * C * sizeof(T) + 4.0 * P * C);
    // an unused wpe (rotary positions) gets a zero gradient: no row t < 0 exists
    hipLaunchKernelGGL(encoder_backward_wpe_kernel<T>, dim3(cdiv((int64_t)P * C, 256)), dim3(256), 0, s, dwpe, dx, B,
                       wpe_used ? T_ : 0, P, C);
    return hipGetLastError();
}

// ============================================================================ AdamW
// "1000 行 C 代码完成 GPT-2 训练的 LLM.c": the step ends with an Adam update.  Decoupled
// weight decay with bias correction (c1 = 1 - beta1^t, c2 = 1 - beta2^t):
//   m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;  p -= lr (m/c1 / (sqrt(v/c2) + eps) + wd p)
// (adamw_one is defined with the embedding backward, which also applies it)

__global__ __launch_bounds__(256) void adamw_kernel(float* p, const float* g, float* m, float* v, bf16* p16,
                                                    int64_t n, float lr, float b1, float b2, float eps, float wd,
                                                    float c1, float c2) {
    const int64_t n4 = n / 4;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        float4 pp = ((float4*)p)[i], gg = ((const float4*)g)[i], mm = ((float4*)m)[i], vv = ((float4*)v)[i];
        adamw_one(pp.x, gg.x, mm.x, vv.x, lr, b1, b2, eps, wd, c1, c2);
        adamw_one(pp.y, gg.y, mm.y, vv.y, lr, b1, b2, eps, wd, c1, c2);
        adamw_one(pp.z, gg.z, mm.z, vv.z, lr, b1, b2, eps, wd, c1, c2);
        adamw_one(pp.w, gg.w, mm.w, vv.w, lr, b1, b2, eps, wd, c1, c2);
        ((float4*)p)[i] = pp;
        ((float4*)m)[i] = mm;
        ((float4*)v)[i] = vv;
        if (p16) {
            uint2 h;
            h.x = pack2_bf16(pp.x, pp.y);
            h.y = pack2_bf16(pp.z, pp.w);
            ((uint2*)p16)[i] = h;
        }
    }
    // tail (n % 4 elements), handled by the first threads of block 0
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        int64_t i = n4 * 4 + threadIdx.x;
        float pp = p[i], mm = m[i], vv = v[i];
        adamw_one(pp, g[i], mm, vv, lr, b1, b2, eps, wd, c1, c2);
        p[i] = pp; m[i] = mm; v[i] = vv;
        if (p16) p16[i] = bf16{f32_to_bf16_bits(pp)};
    }
}

hipError_t adamw(float* p, const float* g, float* m, float* v, bf16* p16, int64_t n, float lr, float b1, float b2,
                 float eps, float wd, float c1, float c2, hipStream_t s) {
    int64_t blocks = (n / 4 + 255) / 256;
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (blocks < 1) blocks = 1;
    ProfScope prof(s, "adamw", 0, (double)n * (28 + (p16 ? 2 : 0)));
    hipLaunchKernelGGL(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, g, m, v, p16, n, lr, b1, b2, eps, wd,
                       c1, c2);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(bf16* out, const float* in, int64_t n) {
    int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) out[i] = bf16{f32_to_bf16_bits(in[i])};
}

hipError_t cast_bf16(bf16* out, const float* in, int64_t n, hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    ProfScope prof(s, "cast_bf16", 0, 6.0 * n);
    hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, in, n);
    return hipGetLastError();
}

// out[i] = sum over k of ws[k * n + i], in split order (deterministic); four
// elements per thread when n % 4 == 0.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(float* out, const float* ws, int splits, int64_t n,
                                                            int64_t ld, bool vec4) {
    const int64_t step = (int64_t)gridDim.x * 256;
    if (vec4) {  // n, ld multiples of 4 and both pointers 16-byte aligned
        const int64_t n4 = n >> 2;
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += step) {
            float4 acc = ((const float4*)ws)[i];
            for (int k = 1; k < splits; ++k) {
                const float4 v = ((const float4*)(ws + (int64_t)k * ld))[i];
                acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
            }
            ((float4*)out)[i] = acc;
        }
        return;
    }
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += step) {
        float acc = 0.f;
        for (int k = 0; k < splits; ++k) acc += ws[(int64_t)k * ld + i];
        out[i] = acc;
    }
}

hipError_t splitk_reduce(float* out, const float* ws, int splits, int64_t n, int64_t stride, hipStream_t s) {
    const bool vec4 = n % 4 == 0 && stride % 4 == 0 && (uintptr_t)out % 16 == 0 && (uintptr_t)ws % 16 == 0;
    int64_t blocks = (vec4 ? n / 4 : n + 255) / 256 + 1;
    if (blocks > 4096) blocks = 4096;
    ProfScope prof(s, "splitk_reduce", 0, 4.0 * (splits + 1) * n);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, out, ws, splits, n, stride,
                       vec4);
    return hipGetLastError();
}

// C[m, n] (bf16, row stride ldc) = bias[n] + sum over k of ws[k][m][n] (dense M x N
// partials), 8 columns per thread; N % 8 == 0.
__global__ __launch_bounds__(256) void splitk_reduce_bf16_kernel(bf16* C, int64_t ldc, const float* ws, int splits,
                                                                 int M, int N, const float* bias) {
    const int cpr = N / 8;
    const int64_t total = (int64_t)M * cpr, mn = (int64_t)M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int m = (int)(i / cpr), n = (int)(i % cpr) * 8;
        const float* p = ws + (int64_t)m * N + n;
        float v[8];
        {
            const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
        for (int k = 1; k < splits; ++k) {
            const float4 a = *(const float4*)(p + k * mn), b = *(const float4*)(p + k * mn + 4);
            v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w; v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
        }
        if (bias) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += bias[n + e];
        }
        st16(C + (int64_t)m * ldc + n, pack16<bf16>(v));
    }
}

hipError_t splitk_reduce_bf16(bf16* C, int64_t ldc, const float* ws, int splits, int M, int N, const float* bias,
                              hipStream_t s) {
    if (N % 8 || ldc % 8) return hipErrorInvalidValue;
    int64_t blocks = ((int64_t)M * (N / 8) + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    ProfScope prof(s, "splitk_reduce_bf16", 0, (4.0 * splits + 2) * M * N);
    hipLaunchKernelGGL(splitk_reduce_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, C, ldc, ws, splits, M, N,
                       bias);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------- instantiations
#define GPT2_INST(T)                                                                                              \
    template hipError_t encoder_forward<T>(T*, const int32_t*, const float*, const float*, int, int, int,        \
                                           hipStream_t, int);                                                     \
    template hipError_t layernorm_forward<T>(T*, float*, const T*, const float*, const float*, int, int,         \
                                             hipStream_t, uint8_t*, int64_t, uint8_t*, bool);                    \
    template hipError_t layernorm_backward<T>(T*, const T*, float*, float*, const T*, const T*, const float*,   \
                                              const float*, int, int, float*, size_t, hipStream_t, bool, uint8_t*,   \
                                              int64_t, uint8_t*);                                                     \
    template hipError_t layernorm_backward_dx<T>(T*, const T*, const T*, const T*, const float*, const float*,   \
                                                 int, int, hipStream_t, bool);                                   \
    template hipError_t layernorm_param_grads<T>(float*, float*, const T*, const T*, const float*, int, int,     \
                                                 float*, size_t, hipStream_t);                                    \
    template hipError_t bias_grad<T>(float*, const T*, int, int, int64_t, float*, size_t, hipStream_t);          \
    template hipError_t crossentropy_fused<T>(T*, float*, const int32_t*, int, int, int64_t, float, hipStream_t,     \
                                              uint8_t*, int64_t, uint8_t*);                                      \
    template hipError_t encoder_backward<T>(float*, float*, const T*, const int32_t*, int, int, int, int, int*,  \
                                            int*, hipStream_t, bool, const AdamwRows&);
GPT2_INST(float)
GPT2_INST(bf16)

}  // namespace gpt2
