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

// Codes of a weight W [R, K] (R outputs, K inputs; bf16, row stride ldw) for both
// products it takes part in: the forward one (blocks of 32 along K: q [R, ldq], scales
// [Kp / 128][R][4]) and, when qt is given, the input-gradient one (blocks of 32 along R,
// i.e. the rows of W^T: qt [K, ldqt], scales [Rp / 128][K][4]).  One block takes a
// 128 x 128 tile of W into LDS (zero outside W) and reads it once for both.
__global__ __launch_bounds__(256) void mx_weight_codes_kernel(const bf16* __restrict__ w, int64_t ldw, int R, int K,
                                                              uint8_t* __restrict__ q, int64_t ldq,
                                                              uint8_t* __restrict__ sq, uint8_t* __restrict__ qt,
                                                              int64_t ldqt, uint8_t* __restrict__ sqt,
                                                              MxWeightStrides bs) {
    __shared__ uint32_t t[128][65];  // 128 rows x 64 words (128 bf16), one word of pad
    const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 128;
    // blockIdx.z: which of a batch of equally shaped weights (one per layer)
    w += blockIdx.z * bs.w;
    q += blockIdx.z * bs.q;
    sq += blockIdx.z * bs.sq;
    if (qt) {
        qt += blockIdx.z * bs.qt;
        sqt += blockIdx.z * bs.sqt;
    }
    // task = 16 * row + chunk: 8 consecutive values; lanes 16j .. 16j + 15 one 128-stage
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int task = threadIdx.x + 256 * i, rr = task >> 4, cc = (task & 15) * 8;
        const int r = r0 + rr, c = c0 + cc;
        const u32x4 raw = (r < R && c < K) ? ld16(w + (int64_t)r * ldw + c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) t[rr][cc / 2 + e] = raw[e];  // K % 8 == 0: a chunk is in or out
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // forward codes: a row's 8 values per task
        const int task = threadIdx.x + 256 * i, rr = task >> 4, cc = (task & 15) * 8;
        float v[8];
        const u32x4 raw = {t[rr][cc / 2], t[rr][cc / 2 + 1], t[rr][cc / 2 + 2], t[rr][cc / 2 + 3]};
        unpack16<bf16>(raw, v);
        uint32_t cw[2];
        const uint32_t word = mx_stage_word(mx_quant8(v, cw));
        const int r = r0 + rr, c = c0 + cc;
        if (r < R) {
            *(uint2*)(q + (int64_t)r * ldq + c) = make_uint2(cw[0], cw[1]);
            if ((task & 15) == 0) *(uint32_t*)(sq + ((int64_t)(c0 / 128) * R + r) * 4) = word;
        }
    }
    if (!qt) return;  // block-uniform
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // transposed codes: a column's 8 values per task
        const int task = threadIdx.x + 256 * i, cc = task >> 4, j = task & 15;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t word = t[8 * j + e][cc >> 1];
            v[e] = __uint_as_float(cc & 1 ? word & 0xffff0000u : word << 16);
        }
        uint32_t cw[2];
        const uint32_t word = mx_stage_word(mx_quant8(v, cw));
        const int k = c0 + cc;
        if (k < K) {
            *(uint2*)(qt + (int64_t)k * ldqt + r0 + 8 * j) = make_uint2(cw[0], cw[1]);
            if (j == 0) *(uint32_t*)(sqt + ((int64_t)(r0 / 128) * K + k) * 4) = word;
        }
    }
}

}  // namespace

hipError_t mx_weight_codes(const bf16* w, int64_t ldw, int R, int K, uint8_t* q, int64_t ldq, uint8_t* sq,
                           uint8_t* qt, int64_t ldqt, uint8_t* sqt, hipStream_t s, int batch,
                           const MxWeightStrides& bs) {
    if (R <= 0 || K <= 0 || batch <= 0) return hipSuccess;
    const int Kp = (K + 127) / 128 * 128, Rp = (R + 127) / 128 * 128;
    if (K % 8 || ldw < K || ldw % 8 || ldq < Kp || ldq % 16 || (qt && (ldqt < Rp || ldqt % 16)) || batch > 65535 ||
        (batch > 1 && (bs.w % 8 || bs.q % 16 || bs.sq % 4 || (qt && (bs.qt % 16 || bs.sqt % 4)))))
        return hipErrorInvalidValue;
    ProfScope prof(s, "mx_weight_codes", 0.0,
                   batch * ((double)R * K * 2 + ((double)R * Kp + (qt ? (double)K * Rp : 0.0)) * (1 + 1 / 32.)));
    hipLaunchKernelGGL(mx_weight_codes_kernel, dim3(Kp / 128, Rp / 128, batch), dim3(256), 0, s, w, ldw, R, K, q, ldq,
                       sq, qt, ldqt, sqt, bs);
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
