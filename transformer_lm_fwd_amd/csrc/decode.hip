// Kernels of incremental generation with a key/value cache (gfx950, bf16).
//
// "GPT-2ベースの3000バイトCで実装されたChatGPTクローン", KVキャッシュ方式: once the first N
// tokens have been run, the (N+1)-th needs only its own row; everything the earlier rows
// produced stays where it was written.  A decode step therefore runs one row per
// sequence through every layer: the matrix products become skinny (a handful of rows
// against a full weight matrix, bound by reading the weights), and attention is one
// query against the cached keys and values of its sequence.
#include <algorithm>

#include "kernels.h"

namespace gpt2 {

// ============================================================================ skinny GEMM
// y[m, n] = epilogue( sum_k x'[m, k] W[n, k] ) for the M <= 16 rows of a decode step,
// W [N, K] row-major (out, in): each output column is one contiguous weight row, and the
// product is bound by reading W once.  On the matrix core: v_mfma_f32_16x16x32_bf16
// with the 16 (zero-padded) rows of x' as A and 16 weight rows as B - lane l supplies
// row / column l % 16 with the 8 k values 8 (l / 16) .. +7, i.e. one 16-byte load of its
// weight row per 32 k, and its accumulators hold column l % 16, rows 4 (l / 16) .. +3.
// Block = NW (8) waves on 16 columns; wave w takes the 32-k steps w, w + NW, .. so the
// weight rows stream in from all waves at once.  x' goes through LDS in chunks of up
// to 2048 k; per chunk a wave first issues its first batch of weight loads (up to 16
// per lane), then every wave - also one with no step in this chunk - takes part in
// staging x' (loads issued eight at a time before their stores), then the wave
// multiplies.  The waves' sums are added through LDS and each thread applies the
// epilogue to one (row, column).
// With LayerNorm gains / shifts, x' = LayerNorm(x): the whole rows are staged (one
// chunk, K <= 2048), each row's mean and rstd (biased variance, eps 1e-5, two passes;
// wave w takes rows w, w + NW, ..) come from LDS, and the rows are normalised in place
// and rounded to bf16 like the forward pass's LayerNorm output.  Every block repeats
// this small prologue, which pays for products with few blocks (qkv, c_fc) but not for
// the lm_head's thousands: that one takes a separately normalised input.
#ifndef SK_NW
#define SK_NW 8  // waves per block
#endif
constexpr int SK_MAXM = 16, SK_KC = 2048, SK_LN_MAXK = 2048, SK_WL = 16;  // weight loads per lane per chunk
constexpr int NW = SK_NW, NT = 64 * SK_NW;

typedef __bf16 sk_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sk_f32x4 __attribute__((ext_vector_type(4)));

template <int EPI, bool LN>
__global__ __launch_bounds__(NT) void skinny_gemm_kernel(SkinnyArgs a) {
    extern __shared__ __attribute__((aligned(16))) bf16 xs[];  // [M][chunk]
    __shared__ float red[NW][16][17];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;
    const int n = blockIdx.x * 16 + col;
    const int KC = LN ? a.K : min(a.K, SK_KC);
    const bf16* wrow = a.W + (int64_t)min(n, a.N - 1) * a.ldw;
    // this thread's epilogue element (row tid / 16, column tid % 16): its bias and
    // residual are requested now, not after the reduction
    const int em = tid >> 4, en = blockIdx.x * 16 + (tid & 15);
    const bool eok = em < a.M && en < a.N;
    const float ebias = (eok && a.bias) ? a.bias[en] : 0.f;
    float eres = 0.f;
    if constexpr (EPI == EPI_BIAS_RES) {
        if (eok) eres = to_f32(a.R[(int64_t)em * a.ldr + en]);
    }
    float gv[8], bv[8];  // LayerNorm gains / shifts of this thread's 8-column chunk (LN: K <= 2048)
    if constexpr (LN) {
        if (8 * tid < a.K) {
#pragma unroll
            for (int e = 0; e < 8; e += 4) {
                *(float4*)&gv[e] = *(const float4*)(a.ln_w + 8 * tid + e);
                *(float4*)&bv[e] = *(const float4*)(a.ln_b + 8 * tid + e);
            }
        }
    }
    sk_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < a.K; k0 += KC) {
        const int kc = min(KC, a.K - k0), cpr = kc / 8, nch = a.M * cpr;
        const int nsteps = (kc + 31) / 32;  // 32-k steps of the chunk; this wave takes w, w + NW, ..
        // this wave's first batch of weight loads (zeros past the chunk: a wave with no
        // 32-k step still takes part in the staging and its barriers)
        u32x4 wv[SK_WL];
        auto load_batch = [&](int sb) {
#pragma unroll
            for (int j = 0; j < SK_WL; ++j) {
                const int kk = 32 * (sb + NW * j) + 8 * kq;
                wv[j] = (n < a.N && kk < kc) ? ld16(wrow + k0 + kk) : u32x4{0u, 0u, 0u, 0u};
            }
        };
        load_batch(w);
        // stage x' while the loads are in flight (every wave, every chunk)
        __syncthreads();  // the previous chunk is no longer read
        for (int b0 = 0; b0 < nch; b0 += NT * 8) {
            u32x4 t[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = b0 + NT * j + tid;
                t[j] = i < nch ? ld16(a.x + (int64_t)(i / cpr) * a.ldx + k0 + (i % cpr) * 8)
                               : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = b0 + NT * j + tid;
                if (i < nch) *(u32x4*)&xs[(i / cpr) * kc + (i % cpr) * 8] = t[j];
            }
        }
        __syncthreads();
        if constexpr (LN) {
            // wave w takes rows w, w + NW, ..: two passes (mean, then the variance about it)
            __shared__ float stat[SK_MAXM][2];
            float part[SK_MAXM / NW], mean[SK_MAXM / NW];
#pragma unroll
            for (int r = 0; r < SK_MAXM / NW; ++r) {
                const int m = w + NW * r;
                part[r] = 0.f;
                if (m < a.M)
                    for (int k = lane * 8; k < kc; k += 512) {
                        float v[8];
                        unpack16<bf16>(*(const u32x4*)(xs + m * kc + k), v);
#pragma unroll
                        for (int e = 0; e < 8; ++e) part[r] += v[e];
                    }
            }
#pragma unroll
            for (int r = 0; r < SK_MAXM / NW; ++r) mean[r] = wave_sum(part[r]) / kc;
#pragma unroll
            for (int r = 0; r < SK_MAXM / NW; ++r) {
                const int m = w + NW * r;
                part[r] = 0.f;
                if (m < a.M)
                    for (int k = lane * 8; k < kc; k += 512) {
                        float v[8];
                        unpack16<bf16>(*(const u32x4*)(xs + m * kc + k), v);
#pragma unroll
                        for (int e = 0; e < 8; ++e) part[r] += (v[e] - mean[r]) * (v[e] - mean[r]);
                    }
            }
#pragma unroll
            for (int r = 0; r < SK_MAXM / NW; ++r) {
                const float var = wave_sum(part[r]) / kc;
                const int m = w + NW * r;
                if (lane == 0 && m < a.M) {
                    stat[m][0] = mean[r];
                    stat[m][1] = 1.0f / sqrtf(var + 1e-5f);
                }
            }
            __syncthreads();
            // thread t normalises the 8-column chunk t of every row
            if (tid < cpr) {
                for (int m = 0; m < a.M; ++m) {
                    float f[8];
                    unpack16<bf16>(*(const u32x4*)&xs[m * kc + 8 * tid], f);
                    const float mu = stat[m][0], rstd = stat[m][1];
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = (f[e] - mu) * rstd * gv[e] + bv[e];
                    *(u32x4*)&xs[m * kc + 8 * tid] = pack16<bf16>(f);
                }
            }
            __syncthreads();
        }
        for (int sb = w; sb < nsteps; sb += NW * SK_WL) {
            if (sb != w) load_batch(sb);
#pragma unroll
            for (int j = 0; j < SK_WL; ++j) {
                const int kk = 32 * (sb + NW * j) + 8 * kq;
                if (32 * (sb + NW * j) < kc) {  // wave-uniform
                    const u32x4 xa = (col < a.M && kk < kc) ? *(const u32x4*)&xs[col * kc + kk] : u32x4{0u, 0u, 0u, 0u};
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(sk_bf16x8, xa),
                                                                  __builtin_bit_cast(sk_bf16x8, wv[j]), acc, 0, 0, 0);
                }
            }
        }
    }
    // acc[i]: row 4 kq + i, column col (of this wave's share of k)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][4 * kq + i][col] = acc[i];
    __syncthreads();
    const int cn = tid & 15;
    float v = 0.f;
    if (eok)
#pragma unroll
        for (int q = 0; q < NW; ++q) v += red[q][em][cn];
    if (!eok) return;
    v += ebias;
    const int64_t o = (int64_t)em * a.ldc + en;
    if constexpr (EPI == EPI_F32) {
        ((float*)a.C)[o] = v;
    } else {
        if constexpr (EPI == EPI_BIAS_RES) v += eres;
        if constexpr (EPI == EPI_BIAS_GELU) {
            if (a.C2) a.C2[o] = from_f32<bf16>(gelu_fwd(v));
        }
        if (a.C) ((bf16*)a.C)[o] = from_f32<bf16>(v);
    }
}

template <bool LN>
static hipError_t skinny_launch(const SkinnyArgs& a, int epi, hipStream_t s) {
    const dim3 grid((a.N + 15) / 16);
    const size_t lds = (size_t)a.M * (LN ? a.K : std::min(a.K, SK_KC)) * 2;
    switch (epi) {
        case EPI_BIAS: hipLaunchKernelGGL((skinny_gemm_kernel<EPI_BIAS, LN>), grid, dim3(NT), lds, s, a); break;
        case EPI_BIAS_RES: hipLaunchKernelGGL((skinny_gemm_kernel<EPI_BIAS_RES, LN>), grid, dim3(NT), lds, s, a); break;
        case EPI_BIAS_GELU: hipLaunchKernelGGL((skinny_gemm_kernel<EPI_BIAS_GELU, LN>), grid, dim3(NT), lds, s, a); break;
        case EPI_F32: hipLaunchKernelGGL((skinny_gemm_kernel<EPI_F32, LN>), grid, dim3(NT), lds, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t skinny_gemm(const SkinnyArgs& a, int epi, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.M > SK_MAXM || a.K % 8 || a.ldx % 8 || a.ldw % 8) return hipErrorInvalidValue;
    if ((a.ln_w != nullptr) != (a.ln_b != nullptr)) return hipErrorInvalidValue;
    if (a.ln_w && (a.K > SK_LN_MAXK || (uintptr_t)a.ln_w % 16 || (uintptr_t)a.ln_b % 16)) return hipErrorInvalidValue;
    ProfScope prof(s, "skinny_gemm", 2.0 * a.M * a.N * a.K,
                   2.0 * a.N * a.K + 2.0 * a.M * a.K + (epi == EPI_F32 ? 4.0 : 2.0) * a.M * a.N);
    return a.ln_w ? skinny_launch<true>(a, epi, s) : skinny_launch<false>(a, epi, s);
}

// ============================================================================ decode attention
// One query per (sequence, head) against cached keys/values 0 .. len-1, head size 64
// ("GPT-2 from scratch with torch", 自注意力: softmax(q k^T / sqrt(hs)) v; the new row sees
// every cached position, so no mask is needed).  Cache rows are the q|k|v rows the
// qkv product wrote, [batch][max_len][3C].  Block (b, h): ADW waves take key chunks of
// 64 in turn.  Lane (g, d8) = (lane / 8, lane % 8) reads 16 bytes (dims 8 d8 ..
// 8 d8 + 7) of the K and V rows of keys g, g + 8, .., so each row is one 128-byte run
// read by eight lanes; a score is summed over those eight lanes by shuffles, and the
// wave keeps a running maximum and sum (online softmax) while each lane adds p v over
// its own keys.  The 8 key groups are combined by shuffles at the end and the waves'
// states are merged through LDS.  (Splitting long contexts over several blocks per
// (sequence, head), with a kernel merging the blocks' softmax states, measured no faster
// at batch 1 and slower at batch 8: the kernel is bound by its memory round trips, not by
// the number of blocks.)
constexpr int ADW = 8;  // waves per (sequence, head) block
__global__ __launch_bounds__(64 * ADW) void attn_decode64_kernel(bf16* y, const bf16* cache, int len, int C, int NH,
                                                                 int64_t bstride) {
    constexpr int HS = 64;
    const int b = blockIdx.x / NH, h = blockIdx.x % NH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int kg = lane >> 3, d8 = lane & 7;
    const int64_t C3 = 3 * (int64_t)C;
    const bf16* base = cache + (int64_t)b * bstride;
    const float c = 0.125f * 1.4426950408889634f;  // 1/sqrt(64) in log2 units
    // lane (kg, d8) owns dims 8 d8 .. 8 d8 + 7 of keys k0 + kg + 8 i (i < 8): eight lanes
    // read one 128-byte K or V row together, and a key's score is summed over its eight
    // lanes, which then all hold it, next to the V row it weighs.
    float qf[8];
    unpack16<bf16>(ld16(base + (int64_t)(len - 1) * C3 + h * HS + 8 * d8), qf);
    float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    for (int k0 = 64 * w; k0 < len; k0 += 64 * ADW) {
        u32x4 kr[8], vr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int key = k0 + kg + 8 * i;
            const bf16* row = base + (int64_t)key * C3 + C + h * HS + 8 * d8;
            kr[i] = key < len ? ld16(row) : u32x4{0u, 0u, 0u, 0u};
            vr[i] = key < len ? ld16(row + C) : u32x4{0u, 0u, 0u, 0u};
        }
        float s[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float kv[8];
            unpack16<bf16>(kr[i], kv);
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = __builtin_fmaf(qf[e], kv[e], dot);
            s[i] = dot;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] += __shfl_xor(s[i], 1, 64);
            s[i] += __shfl_xor(s[i], 2, 64);
            s[i] += __shfl_xor(s[i], 4, 64);
        }
        float smax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[i] = k0 + kg + 8 * i < len ? s[i] * c : -INFINITY;
            smax = fmaxf(smax, s[i]);
        }
        const float mn = fmaxf(m, wave_max(smax));  // finite: key k0 < len
        const float corr = __builtin_amdgcn_exp2f(m - mn);  // m = -inf at first: corr = 0
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= corr;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[i] - mn);  // 0 for keys past len
            psum += p;
            float v[8];
            unpack16<bf16>(vr[i], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(p, v[e], o[e]);
        }
        l = l * corr + psum;
        m = mn;
    }
    // the 8 key groups (lanes d8, d8 + 8, ..) hold partial sums of the same dims
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 8, 64);
        o[e] += __shfl_xor(o[e], 16, 64);
        o[e] += __shfl_xor(o[e], 32, 64);
    }
    l = wave_sum(l) * 0.125f;  // each key's weight was counted by its eight lanes
    __shared__ float sm[ADW], sl[ADW], so[ADW][HS];
    if (lane == 0) {
        sm[w] = m;
        sl[w] = l;
    }
    if (kg == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) so[w][8 * d8 + e] = o[e];
    }
    __syncthreads();
    if (w == 0) {
        float M = sm[0];
#pragma unroll
        for (int i = 1; i < ADW; ++i) M = fmaxf(M, sm[i]);
        float L = 0.f, O = 0.f;
#pragma unroll
        for (int i = 0; i < ADW; ++i) {
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
    hipLaunchKernelGGL(attn_decode64_kernel, dim3(batch * NH), dim3(64 * ADW), 0, s, y, cache, len, C, NH, bstride);
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
