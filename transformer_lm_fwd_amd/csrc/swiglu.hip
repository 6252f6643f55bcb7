// SwiGLU MLP of the Llama-style block ("1000 行 C 代码完成 GPT-2 训练的 LLM.c": the layers
// to add for Llama-2-type models): h = silu(x W_gate^T) * (x W_up^T), silu(g) = g sigmoid(g).
// The gate and up weights are interleaved by row, so the one product x W_gu^T leaves
// (g_j, u_j) in adjacent columns 2j, 2j+1 and a thread's 16-byte loads hold whole pairs.
// Backward: dg = dh u silu'(g), du = dh silu(g), silu'(g) = s (1 + g (1 - s)), s = sigmoid(g).
#include "kernels.h"

namespace gpt2 {

namespace {

__device__ __forceinline__ float sigmoidf(float g) { return 1.f / (1.f + __expf(-g)); }

// Thread: 8 hidden units of a row (16 gate/up values in, 8 out).
template <class T>
__global__ __launch_bounds__(256) void swiglu_forward_kernel(T* __restrict__ h, const T* __restrict__ gu, int N, int H) {
    constexpr int KV = Vec16<T>::N;
    const int cpr = H / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)N * cpr) return;
    const int r = (int)(idx / cpr), j0 = (int)(idx % cpr) * 8;
    const T* src = gu + (int64_t)r * 2 * H + 2 * j0;
    float v[16], o[8];
#pragma unroll
    for (int q = 0; q < 16 / KV; ++q) unpack16<T>(ld16(src + q * KV), v + q * KV);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float g = v[2 * e], u = v[2 * e + 1];
        o[e] = g * sigmoidf(g) * u;
    }
    T* dst = h + (int64_t)r * H + j0;
#pragma unroll
    for (int q = 0; q < 8 / KV; ++q) st16(dst + q * KV, pack16<T>(o + q * KV));
}

template <class T>
__global__ __launch_bounds__(256) void swiglu_backward_kernel(T* __restrict__ dgu, const T* __restrict__ dh,
                                                              const T* __restrict__ gu, int N, int H) {
    constexpr int KV = Vec16<T>::N;
    const int cpr = H / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)N * cpr) return;
    const int r = (int)(idx / cpr), j0 = (int)(idx % cpr) * 8;
    const T* src = gu + (int64_t)r * 2 * H + 2 * j0;
    float v[16], d[8], o[16];
#pragma unroll
    for (int q = 0; q < 16 / KV; ++q) unpack16<T>(ld16(src + q * KV), v + q * KV);
#pragma unroll
    for (int q = 0; q < 8 / KV; ++q) unpack16<T>(ld16(dh + (int64_t)r * H + j0 + q * KV), d + q * KV);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float g = v[2 * e], u = v[2 * e + 1], sg = sigmoidf(g);
        o[2 * e] = d[e] * u * sg * (1.f + g * (1.f - sg));
        o[2 * e + 1] = d[e] * g * sg;
    }
    T* dst = dgu + (int64_t)r * 2 * H + 2 * j0;
#pragma unroll
    for (int q = 0; q < 16 / KV; ++q) st16(dst + q * KV, pack16<T>(o + q * KV));
}

}  // namespace

template <class T>
hipError_t swiglu_forward(T* h, const T* gu, int N, int H, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    if (H % 8) return hipErrorInvalidValue;
    ProfScope prof(s, "swiglu_fwd", 0, (double)N * H * 3 * sizeof(T));
    const int64_t threads = (int64_t)N * (H / 8);
    hipLaunchKernelGGL(swiglu_forward_kernel<T>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, h, gu, N, H);
    return hipGetLastError();
}

template <class T>
hipError_t swiglu_backward(T* dgu, const T* dh, const T* gu, int N, int H, hipStream_t s) {
    if (N <= 0) return hipSuccess;
    if (H % 8) return hipErrorInvalidValue;
    ProfScope prof(s, "swiglu_bwd", 0, (double)N * H * 5 * sizeof(T));
    const int64_t threads = (int64_t)N * (H / 8);
    hipLaunchKernelGGL(swiglu_backward_kernel<T>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, dgu, dh, gu,
                       N, H);
    return hipGetLastError();
}

template hipError_t swiglu_forward<float>(float*, const float*, int, int, hipStream_t);
template hipError_t swiglu_forward<bf16>(bf16*, const bf16*, int, int, hipStream_t);
template hipError_t swiglu_backward<float>(float*, const float*, const float*, int, int, hipStream_t);
template hipError_t swiglu_backward<bf16>(bf16*, const bf16*, const bf16*, int, int, hipStream_t);

}  // namespace gpt2
