// Device-side helpers shared by the gfx950 kernels of the GPT-2 training step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt2 {

// bf16 is carried as its 16-bit pattern; arithmetic is always fp32.
struct bf16 {
    uint16_t x;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return __uint_as_float((uint32_t)v.x << 16); }

// fp32 -> bf16, round to nearest, ties to even: the compiler lowers these
// conversions to gfx950's v_cvt_pk_bf16_f32 (two values per instruction).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <class T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return bf16{f32_to_bf16_bits(v)}; }

// Number of elements of T in one 16-byte vector.
template <class T> struct Vec16 { static constexpr int N = 16 / sizeof(T); };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Unpack a 16-byte vector of T into fp32 values.
template <class T> __device__ __forceinline__ void unpack16(const u32x4& v, float* out);
template <> __device__ __forceinline__ void unpack16<float>(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}
template <> __device__ __forceinline__ void unpack16<bf16>(const u32x4& v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(v[i] << 16);
        out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
template <class T> __device__ __forceinline__ u32x4 pack16(const float* in);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(in[i]);
    return v;
}
template <> __device__ __forceinline__ u32x4 pack16<bf16>(const float* in) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = pack2_bf16(in[2 * i], in[2 * i + 1]);
    return v;
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *(u32x4*)p = v; }

// Wavefront (64 lanes) reductions by butterfly shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// GELU, tanh form (the formula quoted in the comment thread of the 3000-byte C
// GPT-2 page): g(x) = x/2 (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))).  The
// identity (1 + tanh u)/2 = 1/(1 + exp(-2u)) = 1/(1 + 2^a), a = -2 u log2(e), turns
// it into one base-2 exponential (v_exp_f32) and one reciprocal (v_rcp_f32, about
// 1 ulp), with a = x (k0 + k1 x^2) evaluated as one multiply-add and a multiply.
// Far in either tail 2^a is 0 or +inf, and g is x or -0, its limits.
#define GPT2_SQRT_2_OVER_PI 0.7978845608028654f
#define GPT2_GELU_K0 (-2.0f * 1.4426950408889634f * GPT2_SQRT_2_OVER_PI)
#define GPT2_GELU_K1 (GPT2_GELU_K0 * 0.044715f)
__device__ __forceinline__ float gelu_fwd(float x) {
    const float a = x * __builtin_fmaf(x * x, GPT2_GELU_K1, GPT2_GELU_K0);
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
}
// d/dx g(x) = s + x s (1 - s) 2 u'(x),  s = 1/(1 + exp(-2u)),
// u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2)  (since (1+tanh u)/2 = s and tanh' = 1 - tanh^2),
// evaluated as s (1 + w q) with w = x (1 - s) = x - s x and q = 2 u'(x).
__device__ __forceinline__ float gelu_bwd(float x) {
    const float x2 = x * x;
    const float a = x * __builtin_fmaf(x2, GPT2_GELU_K1, GPT2_GELU_K0);
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
    const float q = __builtin_fmaf(x2, 2.0f * GPT2_SQRT_2_OVER_PI * 3.0f * 0.044715f, 2.0f * GPT2_SQRT_2_OVER_PI);
    const float w = __builtin_fmaf(-s, x, x);
    return s * __builtin_fmaf(w, q, 1.0f);
}

}  // namespace gpt2
