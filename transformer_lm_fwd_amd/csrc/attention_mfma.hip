// Causal self-attention on MFMA for bf16 operands and head size 64 (gfx950).
//
// Same computation as the row kernels ("GPT-2 from scratch with torch", 自注意力;
// "从头搭建GPT(Andrej Karpathy) 笔记", 直觉上的self-attention and attention中为什么要做
// scaling): S = q k^T / sqrt(64), keys after the query masked, softmax per query,
// O = P V; only the per-query log-sum-exp is kept for the backward pass.
//
// Layout tricks (v_mfma_f32_16x16x32_bf16, wave64):
//  * Scores are computed transposed, S^T = K Q^T, so the accumulator of lane l
//    holds 4 keys of ONE query (column l % 16).  The 16 A-rows of each score tile
//    are fed a permuted set of keys so that, over two tiles, lane group g = l / 16
//    holds the 8 consecutive keys 8g..8g+7 of a 32-key slice.  Those 8
//    probabilities, packed to bf16, are exactly the B operand of O^T = V^T P^T:
//    no LDS round trip for P.
//  * V (and, in the backward pass, Q, dO, K) is also staged transposed in LDS
//    ([d][key]) so that the matching A/B fragments are single 16-byte reads.
//  * The backward pass is two kernels -- dK/dV over key tiles and dQ over query
//    tiles -- each writing its outputs exactly once, so it needs no atomics and
//    is deterministic.
#include "kernels.h"

namespace gpt2 {
namespace {

constexpr int HS = 64;           // head size handled here
constexpr int TILE = 64;         // queries (or keys) per block
constexpr int PITCH = HS + 8;    // LDS row pitch in bf16 elements (144 bytes)
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t half_of(const u32x4& v, int e) { return (v[e >> 1] >> ((e & 1) * 16)) & 0xffffu; }

// Copies rows [r0, r0+64) (head slice of 64 bf16) of a strided matrix into LDS
// [row][PITCH]; rows >= T are zero.  256 threads, two 16-byte chunks each.
__device__ __forceinline__ void load_rows(bf16* lds, const bf16* g, int64_t ld, int r0, int T, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int c = tid + i * 256;
        int row = c >> 3, dc = c & 7;
        u32x4 v = (r0 + row < T) ? ld16(g + (int64_t)(r0 + row) * ld + dc * 8) : u32x4{0, 0, 0, 0};
        st16(lds + row * PITCH + dc * 8, v);
    }
}

// Same rows stored transposed: lds[d][row].  Thread = (pair of rows, 8 columns).
__device__ __forceinline__ void load_rows_t(bf16* lds, const bf16* g, int64_t ld, int r0, int T, int tid) {
    const int rp = tid >> 3, dc = tid & 7;
    const int ra = r0 + 2 * rp;
    u32x4 v0 = (ra < T) ? ld16(g + (int64_t)ra * ld + dc * 8) : u32x4{0, 0, 0, 0};
    u32x4 v1 = (ra + 1 < T) ? ld16(g + (int64_t)(ra + 1) * ld + dc * 8) : u32x4{0, 0, 0, 0};
    uint32_t* base = (uint32_t*)lds;
#pragma unroll
    for (int e = 0; e < 8; ++e) base[((dc * 8 + e) * PITCH + 2 * rp) >> 1] = half_of(v0, e) | (half_of(v1, e) << 16);
}

// A-row r (0..15) of score tile half `hh` in 32-row slice `sp` maps to row
//   32 sp + 8 (r / 4) + 4 hh + (r % 4),
// so accumulator rows 4g+i of halves 0 and 1 are rows 32 sp + 8 g + (0..7).
__device__ __forceinline__ int perm_row(int sp, int hh, int r) { return 32 * sp + 8 * (r >> 2) + 4 * hh + (r & 3); }

}  // namespace

// ============================================================================ forward
__global__ __launch_bounds__(256) void attn_fwd_mfma64(bf16* out, float* lse, const bf16* qkv, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 sK[TILE * PITCH];
    __shared__ __attribute__((aligned(16))) bf16 sVt[HS * PITCH];
    const int nqt = (T + TILE - 1) / TILE;
    const int qt = nqt - 1 - (int)blockIdx.x;  // longest rows first
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g = lane >> 4;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Qg = base + h * HS;
    const bf16* Kg = base + C + h * HS;
    const bf16* Vg = base + 2 * C + h * HS;
    const int q0 = qt * TILE, qw = q0 + 16 * w, myq = qw + r16;
    const float c = 0.125f * LOG2E;  // 1/sqrt(64), in log2 units

    u32x4 qf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
        qf[kk] = (myq < T) ? ld16(Qg + (int64_t)myq * C3 + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
    f32x4 o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    for (int kt = 0; kt <= qt; ++kt) {
        const int k0 = kt * TILE;
        __syncthreads();
        load_rows(sK, Kg, C3, k0, T, tid);
        load_rows_t(sVt, Vg, C3, k0, T, tid);
        __syncthreads();
        if (qw >= T) continue;
        f32x4 s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int kr = perm_row(j >> 1, j & 1, r16);
            s[j] = mfma(ld16(sK + kr * PITCH + 8 * g), qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
            s[j] = mfma(ld16(sK + kr * PITCH + 32 + 8 * g), qf[1], s[j]);
        }
        const bool edge = (kt == qt) || (k0 + TILE > T);
        float x[16];
        float mt = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = s[2 * sp + (e >> 2)][e & 3] * c;
                const int key = k0 + 32 * sp + 8 * g + e;
                if (edge && (key > myq || key >= T)) v = -INFINITY;
                x[sp * 8 + e] = v;
                mt = fmaxf(mt, v);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float mn = fmaxf(m, mt);
        const float corr = fast_exp2(m - mn);
        l *= corr;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] *= corr;
        u32x4 pk[2];
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(x[sp * 8 + e] - mn);
                l += p[e];
            }
            pk[sp] = pack16<bf16>(p);
        }
        m = mn;
#pragma unroll
        for (int sp = 0; sp < 2; ++sp)
#pragma unroll
            for (int j = 0; j < 4; ++j) o[j] = mfma(ld16(sVt + (16 * j + r16) * PITCH + 32 * sp + 8 * g), pk[sp], o[j]);
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (myq < T) {
        const float inv = 1.0f / l;
        bf16* y = out + ((int64_t)b * T + myq) * C + h * HS;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint2 v;
            v.x = (uint32_t)f32_to_bf16_bits(o[j][0] * inv) | ((uint32_t)f32_to_bf16_bits(o[j][1] * inv) << 16);
            v.y = (uint32_t)f32_to_bf16_bits(o[j][2] * inv) | ((uint32_t)f32_to_bf16_bits(o[j][3] * inv) << 16);
            *(uint2*)(y + 16 * j + 4 * g) = v;
        }
        if (g == 0) lse[(int64_t)bh * T + myq] = (m + __log2f(l)) / LOG2E;
    }
}

// ============================================================================ backward
// D[b, h, q] = sum_d dO[q, d] O[q, d]  (= sum_k P[q, k] dP[q, k])
__global__ __launch_bounds__(256) void attn_bwd_dsum64(float* dsum, const bf16* dout, const bf16* out, int BT, int T,
                                                       int C, int NH) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, head)
    if (i >= (int64_t)BT * NH) return;
    const int row = (int)(i / NH), h = (int)(i % NH);
    const bf16* a = dout + (int64_t)row * C + h * HS;
    const bf16* o = out + (int64_t)row * C + h * HS;
    float acc = 0.f;
#pragma unroll
    for (int d = 0; d < HS; d += 8) {
        float x[8], y[8];
        unpack16<bf16>(ld16(a + d), x);
        unpack16<bf16>(ld16(o + d), y);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += x[e] * y[e];
    }
    const int b = row / T, t = row % T;
    dsum[((int64_t)b * NH + h) * T + t] = acc;
}

// dK, dV for one tile of 64 keys (16 per wave), looping over the query tiles at
// or after it.  Per 32-query slice: S and dP as [query x key] tiles (A = Q or dO
// rows permuted, B = the wave's K or V fragments), then dV += P^T dO and
// dK += dS^T Q with P^T / dS^T as A operands and dO^T / Q^T from LDS as B.
__global__ __launch_bounds__(256) void attn_bwd_dkdv_mfma64(bf16* dqkv, const bf16* qkv, const bf16* dout,
                                                            const float* lse, const float* dsum, int T, int C,
                                                            int NH) {
    __shared__ __attribute__((aligned(16))) bf16 sQ[TILE * PITCH];
    __shared__ __attribute__((aligned(16))) bf16 sG[TILE * PITCH];
    __shared__ __attribute__((aligned(16))) bf16 sQt[HS * PITCH];
    __shared__ __attribute__((aligned(16))) bf16 sGt[HS * PITCH];
    __shared__ float sL[TILE], sD[TILE];
    const int nqt = (T + TILE - 1) / TILE;
    const int kt = blockIdx.x;  // key tile 0 has the most query tiles: scheduled first
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g = lane >> 4;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Qg = base + h * HS;
    const bf16* Kg = base + C + h * HS;
    const bf16* Vg = base + 2 * C + h * HS;
    const bf16* Gg = dout + (int64_t)b * T * C + h * HS;
    const int k0 = kt * TILE, kw = k0 + 16 * w, mykey = kw + r16;
    const float c = 0.125f * LOG2E;

    u32x4 kf[2], vf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        kf[kk] = (mykey < T) ? ld16(Kg + (int64_t)mykey * C3 + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
        vf[kk] = (mykey < T) ? ld16(Vg + (int64_t)mykey * C3 + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
    }
    f32x4 dk[4], dv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dk[j] = dv[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int qt = kt; qt < nqt; ++qt) {
        const int q0 = qt * TILE;
        __syncthreads();
        load_rows(sQ, Qg, C3, q0, T, tid);
        load_rows(sG, Gg, C, q0, T, tid);
        load_rows_t(sQt, Qg, C3, q0, T, tid);
        load_rows_t(sGt, Gg, C, q0, T, tid);
        if (tid < TILE) {
            const int q = q0 + tid;
            sL[tid] = q < T ? lse[(int64_t)bh * T + q] * LOG2E : 0.f;
            sD[tid] = q < T ? dsum[(int64_t)bh * T + q] : 0.f;
        }
        __syncthreads();
        if (kw >= T) continue;
        const bool edge = (qt == kt) || (q0 + TILE > T);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            f32x4 s2[2], p2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int qr = perm_row(sp, hh, r16);
                s2[hh] = mfma(ld16(sQ + qr * PITCH + 8 * g), kf[0], f32x4{0.f, 0.f, 0.f, 0.f});
                s2[hh] = mfma(ld16(sQ + qr * PITCH + 32 + 8 * g), kf[1], s2[hh]);
                p2[hh] = mfma(ld16(sG + qr * PITCH + 8 * g), vf[0], f32x4{0.f, 0.f, 0.f, 0.f});
                p2[hh] = mfma(ld16(sG + qr * PITCH + 32 + 8 * g), vf[1], p2[hh]);
            }
            float p[8], ds[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int ql = 32 * sp + 8 * g + e;
                float pv = fast_exp2(s2[e >> 2][e & 3] * c - sL[ql]);
                if (edge && (q0 + ql >= T || mykey > q0 + ql)) pv = 0.f;
                p[e] = pv;
                ds[e] = pv * (p2[e >> 2][e & 3] - sD[ql]);
            }
            const u32x4 pp = pack16<bf16>(p), dd = pack16<bf16>(ds);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                dv[j] = mfma(pp, ld16(sGt + (16 * j + r16) * PITCH + 32 * sp + 8 * g), dv[j]);
                dk[j] = mfma(dd, ld16(sQt + (16 * j + r16) * PITCH + 32 * sp + 8 * g), dk[j]);
            }
        }
    }
    // dv[j] / dk[j]: column d = 16 j + r16, rows key kw + 4 g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int key = kw + 4 * g + i;
        if (key < T) {
            bf16* row = dqkv + ((int64_t)b * T + key) * C3 + h * HS;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                row[C + 16 * j + r16] = from_f32<bf16>(dk[j][i] * 0.125f);
                row[2 * C + 16 * j + r16] = from_f32<bf16>(dv[j][i]);
            }
        }
    }
}

// dQ for one tile of 64 queries (16 per wave), looping over key tiles up to the
// diagonal: S^T and dP^T as in the forward pass, dS (query x 8 keys per lane) as
// the A operand of dQ = dS K with K^T from LDS.
__global__ __launch_bounds__(256) void attn_bwd_dq_mfma64(bf16* dqkv, const bf16* qkv, const bf16* dout,
                                                          const float* lse, const float* dsum, int T, int C, int NH) {
    __shared__ __attribute__((aligned(16))) bf16 sK[TILE * PITCH];
    __shared__ __attribute__((aligned(16))) bf16 sV[TILE * PITCH];
    __shared__ __attribute__((aligned(16))) bf16 sKt[HS * PITCH];
    const int nqt = (T + TILE - 1) / TILE;
    const int qt = nqt - 1 - (int)blockIdx.x;
    const int bh = blockIdx.y, b = bh / NH, h = bh % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r16 = lane & 15, g = lane >> 4;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = qkv + (int64_t)b * T * C3;
    const bf16* Qg = base + h * HS;
    const bf16* Kg = base + C + h * HS;
    const bf16* Vg = base + 2 * C + h * HS;
    const bf16* Gg = dout + (int64_t)b * T * C + h * HS;
    const int q0 = qt * TILE, qw = q0 + 16 * w, myq = qw + r16;
    const float c = 0.125f * LOG2E;

    u32x4 qf[2], gf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        qf[kk] = (myq < T) ? ld16(Qg + (int64_t)myq * C3 + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
        gf[kk] = (myq < T) ? ld16(Gg + (int64_t)myq * C + 32 * kk + 8 * g) : u32x4{0, 0, 0, 0};
    }
    const float L2 = (myq < T) ? lse[(int64_t)bh * T + myq] * LOG2E : 0.f;
    const float Dq = (myq < T) ? dsum[(int64_t)bh * T + myq] : 0.f;
    f32x4 dq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dq[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int kt = 0; kt <= qt; ++kt) {
        const int k0 = kt * TILE;
        __syncthreads();
        load_rows(sK, Kg, C3, k0, T, tid);
        load_rows(sV, Vg, C3, k0, T, tid);
        load_rows_t(sKt, Kg, C3, k0, T, tid);
        __syncthreads();
        if (qw >= T) continue;
        const bool edge = (kt == qt) || (k0 + TILE > T);
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) {
            f32x4 s2[2], p2[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int kr = perm_row(sp, hh, r16);
                s2[hh] = mfma(ld16(sK + kr * PITCH + 8 * g), qf[0], f32x4{0.f, 0.f, 0.f, 0.f});
                s2[hh] = mfma(ld16(sK + kr * PITCH + 32 + 8 * g), qf[1], s2[hh]);
                p2[hh] = mfma(ld16(sV + kr * PITCH + 8 * g), gf[0], f32x4{0.f, 0.f, 0.f, 0.f});
                p2[hh] = mfma(ld16(sV + kr * PITCH + 32 + 8 * g), gf[1], p2[hh]);
            }
            float ds[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = k0 + 32 * sp + 8 * g + e;
                float pv = fast_exp2(s2[e >> 2][e & 3] * c - L2);
                if (edge && (key > myq || key >= T)) pv = 0.f;
                ds[e] = pv * (p2[e >> 2][e & 3] - Dq);
            }
            const u32x4 dd = pack16<bf16>(ds);
#pragma unroll
            for (int j = 0; j < 4; ++j) dq[j] = mfma(dd, ld16(sKt + (16 * j + r16) * PITCH + 32 * sp + 8 * g), dq[j]);
        }
    }
    // dq[j]: column d = 16 j + r16, rows query qw + 4 g + i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = qw + 4 * g + i;
        if (q < T) {
            bf16* row = dqkv + ((int64_t)b * T + q) * C3 + h * HS;
#pragma unroll
            for (int j = 0; j < 4; ++j) row[16 * j + r16] = from_f32<bf16>(dq[j][i] * 0.125f);
        }
    }
}

// ============================================================================ launchers
hipError_t attention_forward_mfma64(bf16* out, float* lse, const bf16* qkv, int B, int T, int C, int NH,
                                    hipStream_t s) {
    const double pairs = (double)B * NH * T * (T + 1) / 2;
    ProfScope prof(s, "attn_fwd_mfma64", 4.0 * HS * pairs, 2.0 * B * T * NH * HS * 4 + 4.0 * B * NH * T);
    dim3 grid((T + TILE - 1) / TILE, B * NH);
    hipLaunchKernelGGL(attn_fwd_mfma64, grid, dim3(256), 0, s, out, lse, qkv, T, C, NH);
    return hipGetLastError();
}

hipError_t attention_backward_mfma64(bf16* dqkv, float* dsum, const bf16* dout, const bf16* out, const bf16* qkv,
                                     const float* lse, int B, int T, int C, int NH, hipStream_t s) {
    const double pairs = (double)B * NH * T * (T + 1) / 2, io = 2.0 * B * T * NH * HS;
    {
        ProfScope prof(s, "attn_bwd_dsum64", 0, 2 * io + 4.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dsum64, dim3((B * T * NH + 255) / 256), dim3(256), 0, s, dsum, dout, out, B * T,
                           T, C, NH);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((T + TILE - 1) / TILE, B * NH);
    {
        ProfScope prof(s, "attn_bwd_dkdv_mfma64", 4.0 * HS * pairs, 6 * io + 8.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dkdv_mfma64, grid, dim3(256), 0, s, dqkv, qkv, dout, lse, dsum, T, C, NH);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    {
        ProfScope prof(s, "attn_bwd_dq_mfma64", 4.0 * HS * pairs, 5 * io + 8.0 * B * NH * T);
        hipLaunchKernelGGL(attn_bwd_dq_mfma64, grid, dim3(256), 0, s, dqkv, qkv, dout, lse, dsum, T, C, NH);
    }
    return hipGetLastError();
}

}  // namespace gpt2
