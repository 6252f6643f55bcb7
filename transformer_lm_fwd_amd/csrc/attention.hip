// Causal multi-head self-attention, forward and backward (gfx950).
//
// "GPT-2 from scratch with torch", 自注意力: q, k, v are the three C-wide column
// blocks of the fused c_attn output, split into heads of hs = C/NH columns;
// scores q.k are scaled by 1/sqrt(hs) ("从头搭建GPT(Andrej Karpathy) 笔记",
// attention中为什么要做scaling), masked so a position sees only itself and the
// past, soft-maxed per row, and used to average v; heads are written side by side.
//
// This file holds the row-per-thread kernels: one lane owns one query (or key)
// row, K/V (or Q/dO) tiles of 64 rows are staged in LDS, and the softmax is
// computed online so no T x T matrix is stored; only the per-row log-sum-exp is
// kept for the backward pass, which recomputes the probabilities from it.
#include "kernels.h"

namespace gpt2 {

static inline int cdiv_i(int a, int b) { return (a + b - 1) / b; }

template <class T, int HS>
__device__ __forceinline__ void load_row(float* dst, const T* src) {
#pragma unroll
    for (int d = 0; d < HS; d += Vec16<T>::N) unpack16<T>(ld16(src + d), dst + d);
}

// ---------------------------------------------------------------------------- forward
template <class T, int HS>
__global__ __launch_bounds__(64) void attn_fwd_rows(T* out, float* lse, const T* qkv, int T_, int C, int NH) {
    constexpr int TILE = 64, SUB = 16;
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int t = blockIdx.y * TILE + threadIdx.x;
    const int64_t C3 = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * T_ * C3;
    __shared__ float sk[TILE][HS + 1], sv[TILE][HS + 1];
    const float scale = 1.0f / sqrtf((float)HS);

    float q[HS], o[HS];
    float m = -INFINITY, l = 0.f;
    if (t < T_) load_row<T, HS>(q, base + (int64_t)t * C3 + h * HS);
#pragma unroll
    for (int d = 0; d < HS; ++d) o[d] = 0.f;

    const int t_last = min(T_ - 1, (int)blockIdx.y * TILE + TILE - 1);
    for (int k0 = 0; k0 <= t_last; k0 += TILE) {
        __syncthreads();
        {
            int u = k0 + threadIdx.x;
            float kr[HS], vr[HS];
            if (u < T_) {
                load_row<T, HS>(kr, base + (int64_t)u * C3 + C + h * HS);
                load_row<T, HS>(vr, base + (int64_t)u * C3 + 2 * C + h * HS);
            } else {
#pragma unroll
                for (int d = 0; d < HS; ++d) kr[d] = vr[d] = 0.f;
            }
#pragma unroll
            for (int d = 0; d < HS; ++d) { sk[threadIdx.x][d] = kr[d]; sv[threadIdx.x][d] = vr[d]; }
        }
        __syncthreads();
        if (t >= T_) continue;
        for (int j0 = 0; j0 < TILE; j0 += SUB) {
            float s[SUB];
            float mt = -INFINITY;
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                int u = k0 + j0 + j;
                float acc = 0.f;
#pragma unroll
                for (int d = 0; d < HS; ++d) acc += q[d] * sk[j0 + j][d];
                s[j] = (u <= t) ? acc * scale : -INFINITY;
                mt = fmaxf(mt, s[j]);
            }
            if (mt == -INFINITY) continue;
            const float mn = fmaxf(m, mt);
            const float corr = __expf(m - mn);
            l *= corr;
#pragma unroll
            for (int d = 0; d < HS; ++d) o[d] *= corr;
#pragma unroll
            for (int j = 0; j < SUB; ++j) {
                float p = __expf(s[j] - mn);
                l += p;
#pragma unroll
                for (int d = 0; d < HS; ++d) o[d] += p * sv[j0 + j][d];
            }
            m = mn;
        }
    }
    if (t < T_) {
        const float inv = 1.0f / l;
        T* y = out + ((int64_t)b * T_ + t) * C + h * HS;
#pragma unroll
        for (int d = 0; d < HS; d += Vec16<T>::N) {
            float tmp[Vec16<T>::N];
#pragma unroll
            for (int e = 0; e < Vec16<T>::N; ++e) tmp[e] = o[d + e] * inv;
            st16(y + d, pack16<T>(tmp));
        }
        lse[((int64_t)b * NH + h) * T_ + t] = m + __logf(l);
    }
}

// ---------------------------------------------------------------------------- backward
// With P = softmax(S) recomputed from the saved log-sum-exp, S = q.k / sqrt(hs):
//   dV = P^T dO,  dP = dO V^T,  D_t = rowsum(dO_t * O_t) = sum_u P_tu dP_tu,
//   dS = P * (dP - D),  dQ = dS K / sqrt(hs),  dK = dS^T Q / sqrt(hs).

// dQ (and D) : one lane per query row, key tiles in LDS.
template <class T, int HS>
__global__ __launch_bounds__(64) void attn_bwd_dq_rows(T* dqkv, float* dsum, const T* dout, const T* out,
                                                       const T* qkv, const float* lse, int T_, int C, int NH) {
    constexpr int TILE = 64;
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int t = blockIdx.y * TILE + threadIdx.x;
    const int64_t C3 = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * T_ * C3;
    __shared__ float sk[TILE][HS + 1], sv[TILE][HS + 1];
    const float scale = 1.0f / sqrtf((float)HS);

    float q[HS], g[HS], dq[HS];
    float D = 0.f, L = 0.f;
    if (t < T_) {
        load_row<T, HS>(q, base + (int64_t)t * C3 + h * HS);
        load_row<T, HS>(g, dout + ((int64_t)b * T_ + t) * C + h * HS);
        float o[HS];
        load_row<T, HS>(o, out + ((int64_t)b * T_ + t) * C + h * HS);
#pragma unroll
        for (int d = 0; d < HS; ++d) D += g[d] * o[d];
        L = lse[((int64_t)b * NH + h) * T_ + t];
        dsum[((int64_t)b * NH + h) * T_ + t] = D;
    }
#pragma unroll
    for (int d = 0; d < HS; ++d) dq[d] = 0.f;

    const int t_last = min(T_ - 1, (int)blockIdx.y * TILE + TILE - 1);
    for (int k0 = 0; k0 <= t_last; k0 += TILE) {
        __syncthreads();
        {
            int u = k0 + threadIdx.x;
            float kr[HS], vr[HS];
            if (u < T_) {
                load_row<T, HS>(kr, base + (int64_t)u * C3 + C + h * HS);
                load_row<T, HS>(vr, base + (int64_t)u * C3 + 2 * C + h * HS);
            } else {
#pragma unroll
                for (int d = 0; d < HS; ++d) kr[d] = vr[d] = 0.f;
            }
#pragma unroll
            for (int d = 0; d < HS; ++d) { sk[threadIdx.x][d] = kr[d]; sv[threadIdx.x][d] = vr[d]; }
        }
        __syncthreads();
        if (t >= T_) continue;
        const int jmax = min(TILE, t - k0 + 1);
        for (int j = 0; j < jmax; ++j) {
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int d = 0; d < HS; ++d) { s += q[d] * sk[j][d]; dp += g[d] * sv[j][d]; }
            float p = __expf(s * scale - L);
            float ds = p * (dp - D) * scale;
#pragma unroll
            for (int d = 0; d < HS; ++d) dq[d] += ds * sk[j][d];
        }
    }
    if (t < T_) {
        T* dst = dqkv + ((int64_t)b * T_ + t) * C3 + h * HS;
#pragma unroll
        for (int d = 0; d < HS; d += Vec16<T>::N) st16(dst + d, pack16<T>(dq + d));
    }
}

// dK and dV : one lane per key row, query tiles (q, dO, lse, D) in LDS.
// WANT_DK selects which of the two this launch produces (keeps registers low).
template <class T, int HS, bool WANT_DK>
__global__ __launch_bounds__(64) void attn_bwd_dkv_rows(T* dqkv, const float* dsum, const T* dout, const T* qkv,
                                                        const float* lse, int T_, int C, int NH) {
    constexpr int TILE = 64;
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int u = blockIdx.y * TILE + threadIdx.x;
    const int64_t C3 = 3 * (int64_t)C;
    const T* base = qkv + (int64_t)b * T_ * C3;
    __shared__ float sq[TILE][HS + 1], sg[TILE][HS + 1], sl[TILE], sd[TILE];
    const float scale = 1.0f / sqrtf((float)HS);

    float k[HS], acc[HS];
    float v[WANT_DK ? HS : 1];
    if (u < T_) {
        load_row<T, HS>(k, base + (int64_t)u * C3 + C + h * HS);
        if constexpr (WANT_DK) load_row<T, HS>(v, base + (int64_t)u * C3 + 2 * C + h * HS);
    }
#pragma unroll
    for (int d = 0; d < HS; ++d) acc[d] = 0.f;

    const int u_first = blockIdx.y * TILE;
    for (int q0 = (u_first / TILE) * TILE; q0 < T_; q0 += TILE) {
        __syncthreads();
        {
            int t = q0 + threadIdx.x;
            float qr[HS], gr[HS];
            if (t < T_) {
                load_row<T, HS>(qr, base + (int64_t)t * C3 + h * HS);
                load_row<T, HS>(gr, dout + ((int64_t)b * T_ + t) * C + h * HS);
                sl[threadIdx.x] = lse[((int64_t)b * NH + h) * T_ + t];
                sd[threadIdx.x] = dsum[((int64_t)b * NH + h) * T_ + t];
            } else {
#pragma unroll
                for (int d = 0; d < HS; ++d) qr[d] = gr[d] = 0.f;
                sl[threadIdx.x] = 0.f;
                sd[threadIdx.x] = 0.f;
            }
#pragma unroll
            for (int d = 0; d < HS; ++d) { sq[threadIdx.x][d] = qr[d]; sg[threadIdx.x][d] = gr[d]; }
        }
        __syncthreads();
        if (u >= T_) continue;
        const int jbeg = max(0, u - q0), jend = min(TILE, T_ - q0);
        for (int j = jbeg; j < jend; ++j) {
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < HS; ++d) s += sq[j][d] * k[d];
            float p = __expf(s * scale - sl[j]);
            if constexpr (WANT_DK) {
                float dp = 0.f;
#pragma unroll
                for (int d = 0; d < HS; ++d) dp += sg[j][d] * v[d];
                float ds = p * (dp - sd[j]) * scale;
#pragma unroll
                for (int d = 0; d < HS; ++d) acc[d] += ds * sq[j][d];
            } else {
#pragma unroll
                for (int d = 0; d < HS; ++d) acc[d] += p * sg[j][d];
            }
        }
    }
    if (u < T_) {
        T* dst = dqkv + ((int64_t)b * T_ + u) * C3 + (WANT_DK ? C : 2 * C) + h * HS;
#pragma unroll
        for (int d = 0; d < HS; d += Vec16<T>::N) st16(dst + d, pack16<T>(acc + d));
    }
}

template <class T, int HS>
static hipError_t attn_fwd_hs(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s) {
    dim3 grid(B * NH, cdiv_i(T_, 64));
    const double pairs = (double)B * NH * T_ * (T_ + 1) / 2, io = (double)B * T_ * NH * HS * sizeof(T);
    ProfScope prof(s, "attn_fwd_rows", 4.0 * HS * pairs, 4 * io + 4.0 * B * NH * T_);
    hipLaunchKernelGGL((attn_fwd_rows<T, HS>), grid, dim3(64), 0, s, out, lse, qkv, T_, C, NH);
    return hipGetLastError();
}

template <class T, int HS>
static hipError_t attn_bwd_hs(T* dqkv, float* dsum, const T* dout, const T* out, const T* qkv, const float* lse,
                              int B, int T_, int C, int NH, hipStream_t s) {
    dim3 grid(B * NH, cdiv_i(T_, 64));
    const double pairs = (double)B * NH * T_ * (T_ + 1) / 2, io = (double)B * T_ * NH * HS * sizeof(T);
    {
        ProfScope prof(s, "attn_bwd_dq_rows", 4.0 * HS * pairs, 6 * io);
        hipLaunchKernelGGL((attn_bwd_dq_rows<T, HS>), grid, dim3(64), 0, s, dqkv, dsum, dout, out, qkv, lse, T_, C,
                           NH);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(s, "attn_bwd_dv_rows", 2.0 * HS * pairs, 3 * io);
        hipLaunchKernelGGL((attn_bwd_dkv_rows<T, HS, false>), grid, dim3(64), 0, s, dqkv, dsum, dout, qkv, lse, T_, C,
                           NH);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(s, "attn_bwd_dk_rows", 2.0 * HS * pairs, 4 * io);
        hipLaunchKernelGGL((attn_bwd_dkv_rows<T, HS, true>), grid, dim3(64), 0, s, dqkv, dsum, dout, qkv, lse, T_, C,
                           NH);
    }
    return hipGetLastError();
}

template <class T>
hipError_t attention_forward(T* out, float* lse, const T* qkv, int B, int T_, int C, int NH, hipStream_t s,
                             uint8_t* q, int64_t ldq, uint8_t* sc, bool* coded) {
    if (coded) *coded = false;
    if constexpr (sizeof(T) == 2) {
        if (C / NH == 64) {
            const bool codes = q && sc && C % 128 == 0 && ldq >= C && ldq % 16 == 0;
            if (coded) *coded = codes;
            return attention_forward_mfma64(out, lse, qkv, B, T_, C, NH, s, codes ? q : nullptr, ldq,
                                            codes ? sc : nullptr);
        }
    }
    switch (C / NH) {
        case 16: return attn_fwd_hs<T, 16>(out, lse, qkv, B, T_, C, NH, s);
        case 32: return attn_fwd_hs<T, 32>(out, lse, qkv, B, T_, C, NH, s);
        case 64: return attn_fwd_hs<T, 64>(out, lse, qkv, B, T_, C, NH, s);
        case 128: return attn_fwd_hs<T, 128>(out, lse, qkv, B, T_, C, NH, s);
    }
    return hipErrorInvalidValue;
}

template <class T>
hipError_t attention_backward(T* dqkv, float* dsum, const T* dout, const T* out, const T* qkv, const float* lse,
                              int B, int T_, int C, int NH, hipStream_t s) {
    if constexpr (sizeof(T) == 2) {
        if (C / NH == 64) return attention_backward_mfma64(dqkv, dsum, dout, out, qkv, lse, B, T_, C, NH, s);
    }
    switch (C / NH) {
        case 16: return attn_bwd_hs<T, 16>(dqkv, dsum, dout, out, qkv, lse, B, T_, C, NH, s);
        case 32: return attn_bwd_hs<T, 32>(dqkv, dsum, dout, out, qkv, lse, B, T_, C, NH, s);
        case 64: return attn_bwd_hs<T, 64>(dqkv, dsum, dout, out, qkv, lse, B, T_, C, NH, s);
        case 128: return attn_bwd_hs<T, 128>(dqkv, dsum, dout, out, qkv, lse, B, T_, C, NH, s);
    }
    return hipErrorInvalidValue;
}

template hipError_t attention_forward<float>(float*, float*, const float*, int, int, int, int, hipStream_t, uint8_t*,
                                             int64_t, uint8_t*, bool*);
template hipError_t attention_forward<bf16>(bf16*, float*, const bf16*, int, int, int, int, hipStream_t, uint8_t*,
                                            int64_t, uint8_t*, bool*);
template hipError_t attention_backward<float>(float*, float*, const float*, const float*, const float*, const float*,
                                              int, int, int, int, hipStream_t);
template hipError_t attention_backward<bf16>(bf16*, float*, const bf16*, const bf16*, const bf16*, const float*, int,
                                             int, int, int, hipStream_t);

}  // namespace gpt2
