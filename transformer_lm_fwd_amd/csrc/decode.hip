// Kernels of incremental generation with a key/value cache (gfx950, bf16).
//
// "GPT-2ベースの3000バイトCで実装されたChatGPTクローン", KVキャッシュ方式: once the first N
// tokens have been run, the (N+1)-th needs only its own row; everything the earlier rows
// produced stays where it was written.  A decode step therefore runs one row per
// sequence through every layer: the matrix products become skinny (a handful of rows
// against a full weight matrix, bound by reading the weights), and attention is one
// query against the cached keys and values of its sequence.
#include "kernels.h"

namespace gpt2 {

// ============================================================================ skinny GEMM
// y[m, n] = epilogue( sum_k x[m, k] W[n, k] ) for the M <= 16 rows of a decode step.
// W is [N, K] row-major (out, in) - each output column is one contiguous weight row.
// Block: 4 waves; a wave takes 8 columns, 8 lanes per column, and a lane reads 16
// bytes of its row per step, so every column is read as 128-byte segments.  x goes
// through LDS in K chunks of 1024 and is read back 16 bytes at a time (the lanes of
// different columns read the same chunk: a broadcast).  The 8 lanes of a column
// then combine their sums by butterfly shuffles and lane j writes rows j, j + 8.
constexpr int SK_MAXM = 16, SK_KC = 1024;

template <int EPI>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyArgs a) {
    __shared__ __attribute__((aligned(16))) bf16 xs[SK_MAXM][SK_KC];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int gl = lane & 7;
    const int n = (blockIdx.x * 4 + wave) * 8 + (lane >> 3);
    float acc[SK_MAXM];
#pragma unroll
    for (int m = 0; m < SK_MAXM; ++m) acc[m] = 0.f;
    const bf16* wrow = a.W + (int64_t)min(n, a.N - 1) * a.ldw;
    for (int k0 = 0; k0 < a.K; k0 += SK_KC) {
        const int kc = min(SK_KC, a.K - k0), cpr = kc / 8;
        __syncthreads();  // the previous chunk is no longer read
        for (int i = tid; i < a.M * cpr; i += 256) {
            const int m = i / cpr, c = i % cpr;
            *(u32x4*)&xs[m][c * 8] = ld16(a.x + (int64_t)m * a.ldx + k0 + c * 8);
        }
        __syncthreads();
        if (n < a.N) {
            for (int kk = gl * 8; kk < kc; kk += 64) {
                float w8[8];
                unpack16<bf16>(ld16(wrow + k0 + kk), w8);
#pragma unroll
                for (int m = 0; m < SK_MAXM; ++m) {
                    if (m < a.M) {
                        float x8[8];
                        unpack16<bf16>(*(const u32x4*)&xs[m][kk], x8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[m] = __builtin_fmaf(w8[e], x8[e], acc[m]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int m = 0; m < SK_MAXM; ++m) {
        acc[m] += __shfl_xor(acc[m], 1, 64);
        acc[m] += __shfl_xor(acc[m], 2, 64);
        acc[m] += __shfl_xor(acc[m], 4, 64);
    }
    if (n >= a.N) return;
    const float bias = a.bias ? a.bias[n] : 0.f;
#pragma unroll
    for (int r = 0; r < SK_MAXM / 8; ++r) {
        const int m = gl + 8 * r;
        if (m >= a.M) continue;
        // lane gl holds every row's total; pick row m without dynamic register indexing
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < SK_MAXM; ++j)
            if (j == m) v = acc[j];
        v += bias;
        const int64_t o = (int64_t)m * a.ldc + n;
        if constexpr (EPI == EPI_F32) {
            ((float*)a.C)[o] = v;
        } else {
            if constexpr (EPI == EPI_BIAS_RES) v += to_f32(a.R[(int64_t)m * a.ldr + n]);
            if constexpr (EPI == EPI_BIAS_GELU) {
                if (a.C2) a.C2[o] = from_f32<bf16>(gelu_fwd(v));
            }
            if (a.C) ((bf16*)a.C)[o] = from_f32<bf16>(v);
        }
    }
}

hipError_t skinny_gemm(const SkinnyArgs& a, int epi, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.M > SK_MAXM || a.K % 8 || a.ldx % 8 || a.ldw % 8) return hipErrorInvalidValue;
    const dim3 grid((a.N + 31) / 32);
    ProfScope prof(s, "skinny_gemm", 2.0 * a.M * a.N * a.K,
                   2.0 * a.N * a.K + 2.0 * a.M * a.K + (epi == EPI_F32 ? 4.0 : 2.0) * a.M * a.N);
    switch (epi) {
        case EPI_BIAS: hipLaunchKernelGGL(skinny_gemm_kernel<EPI_BIAS>, grid, dim3(256), 0, s, a); break;
        case EPI_BIAS_RES: hipLaunchKernelGGL(skinny_gemm_kernel<EPI_BIAS_RES>, grid, dim3(256), 0, s, a); break;
        case EPI_BIAS_GELU: hipLaunchKernelGGL(skinny_gemm_kernel<EPI_BIAS_GELU>, grid, dim3(256), 0, s, a); break;
        case EPI_F32: hipLaunchKernelGGL(skinny_gemm_kernel<EPI_F32>, grid, dim3(256), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ============================================================================ decode attention
// One query per (sequence, head) against cached keys/values 0 .. len-1, head size 64
// ("GPT-2 from scratch with torch", 自注意力: softmax(q k^T / sqrt(hs)) v; the new row sees
// every cached position, so no mask is needed).  Cache rows are the q|k|v rows the
// qkv product wrote, [batch][max_len][3C].  Block (b, h): 4 waves take key chunks of
// 64 in turn; lane j scores key 64c + j (its key row read as 8 x 16 bytes against the
// query held in registers), the wave keeps a running maximum and sum (online softmax),
// and o[d] (lane = d) adds p_j v_j[d] over the chunk, p_j broadcast by shuffle and
// v_j read as one 128-byte row per key.  The four waves' states are merged through LDS.
__global__ __launch_bounds__(256) void attn_decode64_kernel(bf16* y, const bf16* cache, int len, int C, int NH,
                                                            int64_t bstride) {
    constexpr int HS = 64;
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = cache + (int64_t)b * bstride;
    const float c = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) in log2 units
    u32x4 q[8];
    const bf16* qrow = base + (int64_t)(len - 1) * C3 + h * HS;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = ld16(qrow + 8 * i);
    float m = -INFINITY, l = 0.f, o = 0.f;
    for (int k0 = 64 * w; k0 < len; k0 += 256) {
        const int key = k0 + lane;
        float s = -INFINITY;
        if (key < len) {
            const bf16* krow = base + (int64_t)key * C3 + C + h * HS;
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float kv[8], qv[8];
                unpack16<bf16>(ld16(krow + 8 * i), kv);
                unpack16<bf16>(q[i], qv);
#pragma unroll
                for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qv[e], kv[e], dot);
            }
            s = dot * c;
        }
        const float mn = fmaxf(m, wave_max(s));
        const float corr = __builtin_amdgcn_exp2f(m - mn);  // m = -inf at first: corr = 0
        const float p = key < len ? __builtin_amdgcn_exp2f(s - mn) : 0.f;
        l = l * corr + p;
        o *= corr;
        m = mn;
        const int nk = min(64, len - k0);
        const bf16* vcol = base + (int64_t)k0 * C3 + 2 * C + h * HS + lane;
        for (int j = 0; j < nk; ++j) o = __builtin_fmaf(__shfl(p, j, 64), to_f32(vcol[(int64_t)j * C3]), o);
    }
    l = wave_sum(l);
    __shared__ float sm[4], sl[4], so[4][HS];
    if (lane == 0) {
        sm[w] = m;
        sl[w] = l;
    }
    so[w][lane] = o;
    __syncthreads();
    if (w == 0) {
        float M = sm[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) M = fmaxf(M, sm[i]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float f = sm[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[i] - M);  // waves without keys
            L += sl[i] * f;
            O += so[i][lane] * f;
        }
        y[(int64_t)b * C + h * HS + lane] = from_f32<bf16>(O / L);
    }
}

hipError_t attention_decode(bf16* y, const bf16* cache, int batch, int len, int C, int NH, int64_t bstride,
                            hipStream_t s) {
    if (C / NH != 64 || len < 1) return hipErrorInvalidValue;
    ProfScope prof(s, "attn_decode64", 4.0 * batch * C * len, 4.0 * batch * C * len + 4.0 * batch * C);
    hipLaunchKernelGGL(attn_decode64_kernel, dim3(batch * NH), dim3(256), 0, s, y, cache, len, C, NH, bstride);
    return hipGetLastError();
}

// ============================================================================ logits rows
// out[r, v] = (float) logits[rows[r]... ]: row (r * stride_rows + offset) of a bf16
// [rows][ldl] logits buffer widened into a dense fp32 [R][V] block.
__global__ __launch_bounds__(256) void logits_rows_kernel(float* out, const bf16* logits, int R, int V, int64_t ldl,
                                                          int row_stride, int row_offset) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)R * V) return;
    const int r = (int)(i / V), v = (int)(i % V);
    out[i] = to_f32(logits[((int64_t)r * row_stride + row_offset) * ldl + v]);
}

hipError_t logits_rows(float* out, const bf16* logits, int R, int V, int64_t ldl, int row_stride, int row_offset,
                       hipStream_t s) {
    const int64_t n = (int64_t)R * V;
    ProfScope prof(s, "logits_rows", 0, 6.0 * n);
    hipLaunchKernelGGL(logits_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, out, logits, R, V, ldl,
                       row_stride, row_offset);
    return hipGetLastError();
}

}  // namespace gpt2
