// MX FP8 block quantization in registers, for kernels whose 8-value chunks of a row
// sit in consecutive lanes: lanes 4j .. 4j+3 of a wave hold one 32-value block and
// lanes 16j .. 16j+15 one 128-value k-stage (whose 4 scale bytes leave as one word).
//
// Scale of a block ("1000 行 C 代码完成 GPT-2 训练的 LLM.c": precision below 16 bits, in
// the block-scaled E4M3 format of gfx950's matrix cores): the smallest 2^e with
// amax <= 448 2^e, e clamped to [-127, 127], -127 for an all-zero block.  For a
// normal amax = 1.m 2^E, amax / 2^(E-8) = 1.m 2^8 lies in [256, 512) and exceeds
// 448 = 1.75 2^8 exactly when the mantissa field exceeds 0x600000.  Codes: x 2^-e
// rounded to the nearest E4M3 value, ties to even (v_cvt_pk_fp8_f32).
#pragma once

#include "common.h"

namespace gpt2 {

__device__ __forceinline__ int mx_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (amax == 0.f) return -127;
    const int E = (int)((b >> 23) & 0xFF) - 127;  // a subnormal amax lands far below the clamp
    const int e = E - 8 + ((b & 0x7FFFFF) > 0x600000 ? 1 : 0);
    return e < -127 ? -127 : e > 127 ? 127 : e;
}

// Quantizes this lane's 8 values (all lanes of the wave must call it): the 8 codes in
// q[0..1] and the block's scale byte (e + 127) in the return value.
__device__ __forceinline__ uint32_t mx_quant8(const float* v, uint32_t* q) {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int ex = mx_exponent(amax);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float a0 = __builtin_amdgcn_ldexpf(v[4 * h + 0], -ex), a1 = __builtin_amdgcn_ldexpf(v[4 * h + 1], -ex);
        const float a2 = __builtin_amdgcn_ldexpf(v[4 * h + 2], -ex), a3 = __builtin_amdgcn_ldexpf(v[4 * h + 3], -ex);
        int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
        q[h] = (uint32_t)r;
    }
    return (uint32_t)(ex + 127);
}

// The stage word (scale bytes of blocks 0..3 of a 128-value stage), valid in the
// stage's first lane (lane % 16 == 0); all lanes must call it.
__device__ __forceinline__ uint32_t mx_stage_word(uint32_t sbyte) {
    const uint32_t s1 = __shfl_down(sbyte, 4), s2 = __shfl_down(sbyte, 8), s3 = __shfl_down(sbyte, 12);
    return sbyte | (s1 << 8) | (s2 << 16) | (s3 << 24);
}

// Round-trip through bf16, so that codes made from fp32 values equal those made later
// from the stored bf16 activation.
__device__ __forceinline__ void round_bf16_8(float* v) {
    float t[8];
    unpack16<bf16>(pack16<bf16>(v), t);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = t[e];
}

}  // namespace gpt2
