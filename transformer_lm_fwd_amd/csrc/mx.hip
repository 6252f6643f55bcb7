// MX FP8 quantization: bf16 rows -> E4M3 codes with one shared power-of-two scale
// per 32 consecutive values ("1000 行 C 代码完成 GPT-2 训练的 LLM.c": the precision
// step below 16 bits; the block-scaled E4M3 format is the one gfx950's matrix cores
// take natively, v_mfma_scale_f32_32x32x64_f8f6f4).
//
// Scale of a block with largest magnitude amax: the smallest 2^e with amax <= 448 2^e,
// so nothing is clipped; e is clamped to E8M0's [-127, 127] and an all-zero block
// gets -127.  Elements: x 2^-e rounded to the nearest E4M3 value, ties to the even
// mantissa, by v_cvt_pk_fp8_f32 (gfx950 converts to the OCP E4M3 encoding with the
// rounding mode's round-to-nearest-even).
//
// Layout written (what the MX GEMM streams into LDS): codes [R, Kp] with row stride
// ldq bytes, Kp = K rounded up to 128 and zero codes past K; scales
// [Kp / 128][R][4] bytes, so one k-stage of 128 codes of a run of rows has its
// scales in one contiguous run of 4-byte words.
#include "kernels.h"
#include "mx_quant.h"

namespace gpt2 {

namespace {

// One thread: 8 consecutive values of a row; 4 threads: one block of 32; 16 threads:
// one k-stage of 128 (their scales leave as one 4-byte word).
__global__ __launch_bounds__(256) void mx_quantize_kernel(const bf16* __restrict__ x, int64_t ldx, int R, int K,
                                                          int Kp, uint8_t* __restrict__ q, int64_t ldq,
                                                          uint8_t* __restrict__ sc) {
    const int cpr = Kp / 8;  // chunks per row (a multiple of 16)
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const bool live = idx < (int64_t)R * cpr;  // a whole 16-lane group is live or not
    const int row = live ? (int)(idx / cpr) : 0, c = live ? (int)(idx % cpr) : 0;
    const int k0 = c * 8;
    float v[8];
    if (live && k0 < K) {
        unpack16<bf16>(ld16(x + (int64_t)row * ldx + k0), v);  // K % 8 == 0: all 8 or none
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
    uint32_t w[2];
    const uint32_t word = mx_stage_word(mx_quant8(v, w));
    if (!live) return;
    *(uint2*)(q + (int64_t)row * ldq + k0) = make_uint2(w[0], w[1]);
    if ((c & 15) == 0) *(uint32_t*)(sc + ((int64_t)(c / 16) * R + row) * 4) = word;
}

// y [K, ldy] = x [R, ldx]^T over a 64 x 64 tile per block (through LDS, rows padded
// by 2 elements against bank conflicts); columns R .. Rp - 1 of y are written as zero.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16* __restrict__ x, int64_t ldx, int R, int K,
                                                             bf16* __restrict__ y, int64_t ldy, int Rp) {
    __shared__ uint16_t t[64][66];
    const int r0 = blockIdx.y * 64, k0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4 threads
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = r0 + ty + 4 * i, k = k0 + tx;
        t[ty + 4 * i][tx] = (r < R && k < K) ? x[(int64_t)r * ldx + k].x : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int k = k0 + ty + 4 * i, r = r0 + tx;
        if (k < K && r < Rp) y[(int64_t)k * ldy + r] = bf16{t[tx][ty + 4 * i]};
    }
}

}  // namespace

hipError_t transpose_bf16(const bf16* x, int64_t ldx, int R, int K, bf16* y, int64_t ldy, int Rp, hipStream_t s) {
    if (R <= 0 || K <= 0) return hipSuccess;
    if (ldx < K || Rp < R || ldy < Rp) return hipErrorInvalidValue;
    ProfScope prof(s, "transpose_bf16", 0.0, 2.0 * R * K + 2.0 * K * Rp);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((K + 63) / 64, (Rp + 63) / 64), dim3(256), 0, s, x, ldx, R, K, y,
                       ldy, Rp);
    return hipGetLastError();
}

hipError_t mx_quantize(const bf16* x, int64_t ldx, int R, int K, uint8_t* q, int64_t ldq, uint8_t* sc,
                       hipStream_t s) {
    if (R <= 0 || K <= 0) return hipSuccess;
    const int Kp = (K + 127) / 128 * 128;
    if (K % 8 || ldx < K || ldx % 8 || ldq < Kp || ldq % 16) return hipErrorInvalidValue;
    const int64_t threads = (int64_t)R * (Kp / 8);
    ProfScope prof(s, "mx_quantize", 0.0, (double)R * K * 2 + (double)R * Kp + (double)R * Kp / 32);
    hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, ldx, R, K,
                       Kp, q, ldq, sc);
    return hipGetLastError();
}

}  // namespace gpt2
