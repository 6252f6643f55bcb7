// MFMA-tiled GEMM for gfx950 with the fused epilogues of the GPT-2 step.
//
// Every linear layer of the model is a matrix product plus a bias repeated over
// the rows ("GPT-2ベースの3000バイトCで実装されたChatGPTクローン", ニューラルネットワーク層の実装),
// weights stored (out, in) row-major.  The step needs three operand layouts:
//   forward   Y  = X  W^T : A = X  (k-contiguous), B = W (k-contiguous)
//   dX        dX = dY W   : A = dY (k-contiguous), B = W (n-contiguous)
//   dW        dW = dY^T X : A = dY (m-contiguous), B = X (n-contiguous)
// Tiles are staged through LDS always k-contiguous, so the MFMA fragment reads
// are one 16-byte LDS read per lane in every layout: a k-contiguous operand is
// copied as is, an mn-contiguous one is loaded as KV x KV blocks (KV elements
// per 16 bytes) and transposed in registers on the way to LDS.
//
// MFMA use (wave64): v_mfma_f32_16x16x32_bf16 for bf16 operands and
// v_mfma_f32_16x16x4_f32 for fp32 operands.  Lane l supplies row (l % 16) of
// its 16-row A block and column (l % 16) of its 16-column B block, with a
// group of k values selected by l / 16; the accumulator of lane l holds rows
// 4*(l/16) .. +3 of column l % 16.  The reduction over k does not depend on
// which k a lane group takes as long as A and B agree, so both read the same
// k offsets.
#include <string>

#include "kernels.h"

namespace gpt2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

template <class T> struct MfmaTraits;
template <> struct MfmaTraits<bf16> {
    static constexpr int KSLICE = 32;  // k consumed by one fragment pair
    __device__ static __forceinline__ f32x4 step(const u32x4& a, const u32x4& b, f32x4 acc) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
    }
};
template <> struct MfmaTraits<float> {
    static constexpr int KSLICE = 16;
    __device__ static __forceinline__ f32x4 step(const u32x4& a, const u32x4& b, f32x4 acc) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc, 0, 0, 0);
        return acc;
    }
};

// Transpose a KV x KV block held as KV 16-byte rows (row r = k, element j = mn)
// into KV 16-byte rows indexed by mn holding KV consecutive k.
template <class T> __device__ __forceinline__ void transpose_block(const u32x4* in, u32x4* out);
template <> __device__ __forceinline__ void transpose_block<float>(const u32x4* in, u32x4* out) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) out[j][r] = in[r][j];
}
template <> __device__ __forceinline__ void transpose_block<bf16>(const u32x4* in, u32x4* out) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int w = j >> 1, sh = (j & 1) * 16;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t lo = (in[2 * p][w] >> sh) & 0xffffu;
            uint32_t hi = (in[2 * p + 1][w] >> sh) & 0xffffu;
            out[j][p] = lo | (hi << 16);
        }
    }
}

// Loads one ROWS x BK tile of an operand into registers and stores it to LDS,
// k-contiguous with row pitch PITCH elements.
template <class T, bool KCONTIG, int ROWS, int BK, int NT>
struct TileLoader {
    static constexpr int KV = Vec16<T>::N;
    // k-contiguous: ROWS * BK / KV chunks of 16 bytes
    static constexpr int NCHUNK = ROWS * (BK / KV);
    // mn-contiguous: KV x KV blocks
    static constexpr int NBLK = (BK / KV) * (ROWS / KV);
    static constexpr int NREG = KCONTIG ? (NCHUNK + NT - 1) / NT : ((NBLK + NT - 1) / NT) * KV;
    u32x4 r[NREG];

    // rows: valid rows [0, nrows) of this tile; k range valid [0, kvalid)
    __device__ __forceinline__ void load(const T* base, int64_t ld, int row0, int nrows, int k0, int kend, int tid) {
        if constexpr (KCONTIG) {
#pragma unroll
            for (int i = 0; i < NREG; ++i) {
                int c = tid + i * NT;
                int row = c / (BK / KV), kc = c % (BK / KV);
                int k = k0 + kc * KV;
                bool ok = (c < NCHUNK) && (row0 + row < nrows) && (k < kend);
                r[i] = ok ? ld16(base + (int64_t)(row0 + row) * ld + k) : u32x4{0, 0, 0, 0};
            }
        } else {
#pragma unroll
            for (int i = 0; i < NREG / KV; ++i) {
                int b = tid + i * NT;
                int kb = b / (ROWS / KV), mb = b % (ROWS / KV);
                int mn = row0 + mb * KV;
                bool okb = (b < NBLK) && (mn < nrows);
#pragma unroll
                for (int rr = 0; rr < KV; ++rr) {
                    int k = k0 + kb * KV + rr;
                    bool ok = okb && (k < kend);
                    r[i * KV + rr] = ok ? ld16(base + (int64_t)k * ld + mn) : u32x4{0, 0, 0, 0};
                }
            }
        }
    }
    template <int PITCH>
    __device__ __forceinline__ void store(T* lds, int tid) {
        if constexpr (KCONTIG) {
#pragma unroll
            for (int i = 0; i < NREG; ++i) {
                int c = tid + i * NT;
                if (c < NCHUNK) {
                    int row = c / (BK / KV), kc = c % (BK / KV);
                    st16(lds + row * PITCH + kc * KV, r[i]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NREG / KV; ++i) {
                int b = tid + i * NT;
                if (b < NBLK) {
                    int kb = b / (ROWS / KV), mb = b % (ROWS / KV);
                    u32x4 t[KV];
                    transpose_block<T>(&r[i * KV], t);
#pragma unroll
                    for (int j = 0; j < KV; ++j) st16(lds + (mb * KV + j) * PITCH + kb * KV, t[j]);
                }
            }
        }
    }
};

template <class T, int EPI>
__device__ __forceinline__ void epilogue_store(const GemmArgs& a, float* wsC, int row, int col, float v) {
    if (row >= a.M || col >= a.N) return;
    const int64_t o = (int64_t)row * a.ldc + col;
    if constexpr (EPI == EPI_F32) {
        wsC[o] = v;
    } else {
        T* C = (T*)a.C;
        if constexpr (EPI == EPI_BIAS) {
            if (a.bias) v += a.bias[col];
            C[o] = from_f32<T>(v);
        } else if constexpr (EPI == EPI_BIAS_RES) {
            if (a.bias) v += a.bias[col];
            C[o] = from_f32<T>(to_f32(((const T*)a.R)[o]) + v);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
            if (a.bias) v += a.bias[col];
            C[o] = from_f32<T>(v);
            ((T*)a.C2)[o] = from_f32<T>(gelu_fwd(v));
        } else if constexpr (EPI == EPI_GELU_BWD) {
            C[o] = from_f32<T>(v * gelu_bwd(to_f32(((const T*)a.R)[o])));
        }
    }
}

template <class T, bool AK, bool BKC, int EPI, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs a, int k_per_split, int64_t split_stride) {
    constexpr int NT = 64 * WM * WN;
    constexpr int KV = Vec16<T>::N;
    constexpr int PITCH = BK + KV;
    constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
    constexpr int KSLICE = MfmaTraits<T>::KSLICE;
    constexpr int SA = BM * PITCH, SB = BN * PITCH;
    __shared__ __attribute__((aligned(16))) T lds[2][SA + SB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int kbeg = blockIdx.z * k_per_split;
    const int kend = min(a.K, kbeg + k_per_split);
    const T* A = (const T*)a.A;
    const T* B = (const T*)a.B;

    TileLoader<T, AK, BM, BK, NT> la;
    TileLoader<T, BKC, BN, BK, NT> lb;

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    if (nk > 0) {
        la.load(A, a.lda, m0, a.M, kbeg, kend, tid);
        lb.load(B, a.ldb, n0, a.N, kbeg, kend, tid);
        la.template store<PITCH>(lds[0], tid);
        lb.template store<PITCH>(lds[0] + SA, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            la.load(A, a.lda, m0, a.M, kbeg + (kt + 1) * BK, kend, tid);
            lb.load(B, a.ldb, n0, a.N, kbeg + (kt + 1) * BK, kend, tid);
        }
        const T* sA = lds[cur] + (wm * TM * 16) * PITCH;
        const T* sB = lds[cur] + SA + (wn * TN * 16) * PITCH;
#pragma unroll
        for (int ks = 0; ks < BK / KSLICE; ++ks) {
            const int koff = ks * KSLICE + (lane >> 4) * KV;
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = ld16(sA + (i * 16 + (lane & 15)) * PITCH + koff);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = ld16(sB + (j * 16 + (lane & 15)) * PITCH + koff);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = MfmaTraits<T>::step(fa[i], fb[j], acc[i][j]);
        }
        if (kt + 1 < nk) {
            la.template store<PITCH>(lds[cur ^ 1], tid);
            lb.template store<PITCH>(lds[cur ^ 1] + SA, tid);
        }
        __syncthreads();
    }

    float* wsC = nullptr;
    if constexpr (EPI == EPI_F32) wsC = (float*)a.C + (int64_t)blockIdx.z * split_stride;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                int row = m0 + wm * TM * 16 + i * 16 + (lane >> 4) * 4 + r;
                int col = n0 + wn * TN * 16 + j * 16 + (lane & 15);
                epilogue_store<T, EPI>(a, wsC, row, col, acc[i][j][r]);
            }
}

template <class T, bool AK, bool BKC, int EPI>
static const char* gemm_name() {
    static const std::string n = std::string("gemm_") + (sizeof(T) == 2 ? "bf16_" : "f32_") +
                                 (AK && BKC ? "xwT" : AK ? "dyW" : "dyTx") + "_" +
                                 (EPI == EPI_BIAS ? "bias" : EPI == EPI_BIAS_RES ? "bias_res" :
                                  EPI == EPI_BIAS_GELU ? "bias_gelu" : EPI == EPI_GELU_BWD ? "gelu_bwd" : "f32out");
    return n.c_str();
}

template <class T, bool AK, bool BKC, int EPI>
static hipError_t launch(const GemmArgs& a, int splits, int k_per_split, int64_t split_stride, hipStream_t s) {
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2;
    constexpr int BK = sizeof(T) == 2 ? 64 : 32;
    dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM, splits);
    const double es = sizeof(T), mn = (double)a.M * a.N;
    const double out_bytes = EPI == EPI_F32 ? 4 * mn : (EPI == EPI_BIAS ? es * mn : 2 * es * mn);
    ProfScope prof(s, gemm_name<T, AK, BKC, EPI>(), 2.0 * mn * a.K, es * ((double)a.M + a.N) * a.K + out_bytes);
    hipLaunchKernelGGL((gemm_kernel<T, AK, BKC, EPI, BM, BN, BK, WM, WN>), grid, dim3(64 * WM * WN), 0, s, a,
                       k_per_split, split_stride);
    return hipGetLastError();
}

template <class T, int EPI>
static hipError_t dispatch_layout(const GemmArgs& a, bool ak, bool bk, int splits, int kps, int64_t ss,
                                  hipStream_t s) {
    if (ak && bk) return launch<T, true, true, EPI>(a, splits, kps, ss, s);
    if (ak && !bk) return launch<T, true, false, EPI>(a, splits, kps, ss, s);
    if (!ak && !bk) return launch<T, false, false, EPI>(a, splits, kps, ss, s);
    return hipErrorInvalidValue;  // (m-contiguous A, k-contiguous B) is not used by the step
}

template <class T>
hipError_t gemm(const GemmArgs& a, bool ak, bool bk, int epi, float* ws, size_t ws_floats, hipStream_t s) {
    constexpr int BK = sizeof(T) == 2 ? 64 : 32;
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (epi == EPI_F32) {
        // Output fp32 [M, N] with row stride ldc.  Few output tiles and a long K:
        // split K over blockIdx.z into fp32 partials in `ws`, then reduce in a fixed order.
        int tiles = ((a.M + 127) / 128) * ((a.N + 127) / 128);
        int splits = 1;
        if (ws && a.ldc == a.N) {
            while (splits < 16 && tiles * splits < 512 && a.K / (splits * 2) >= 8 * BK &&
                   (size_t)(splits * 2) * a.M * a.N <= ws_floats)
                splits *= 2;
        }
        if (splits == 1) return dispatch_layout<T, EPI_F32>(a, ak, bk, 1, a.K, 0, s);
        int kps = (a.K + splits - 1) / splits;
        kps = (kps + BK - 1) / BK * BK;
        splits = (a.K + kps - 1) / kps;
        GemmArgs p = a;
        p.C = ws;
        hipError_t e = dispatch_layout<T, EPI_F32>(p, ak, bk, splits, kps, (int64_t)a.M * a.N, s);
        if (e != hipSuccess) return e;
        return splitk_reduce((float*)a.C, ws, splits, (int64_t)a.M * a.N, s);
    }
    switch (epi) {
        case EPI_BIAS: return dispatch_layout<T, EPI_BIAS>(a, ak, bk, 1, a.K, 0, s);
        case EPI_BIAS_RES: return dispatch_layout<T, EPI_BIAS_RES>(a, ak, bk, 1, a.K, 0, s);
        case EPI_BIAS_GELU: return dispatch_layout<T, EPI_BIAS_GELU>(a, ak, bk, 1, a.K, 0, s);
        case EPI_GELU_BWD: return dispatch_layout<T, EPI_GELU_BWD>(a, ak, bk, 1, a.K, 0, s);
    }
    return hipErrorInvalidValue;
}

template hipError_t gemm<float>(const GemmArgs&, bool, bool, int, float*, size_t, hipStream_t);
template hipError_t gemm<bf16>(const GemmArgs&, bool, bool, int, float*, size_t, hipStream_t);

}  // namespace gpt2
