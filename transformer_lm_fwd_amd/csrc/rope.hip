// Rotary position embedding ("GPT-2 from scratch with torch", token and position
// embedding: RoPE, Su et al. 2021, as the newer alternative to learned position
// vectors), in RoFormer's form: the pair (x[2i], x[2i+1]) of a query or key head at
// position m is turned by m theta_i, theta_i = base^(-2i / hs).  It replaces wpe: the
// encoder adds no position row and wpe keeps a zero gradient.
//
// The cos / sin table [max_seq_len][hs / 2] is built once in float64 and rounded to
// fp32.  The turn is done in place on the q | k columns of the qkv rows after the
// qkv product (forward, and for each decode row), and turned back on the gradients
// the attention backward leaves there.
#include <algorithm>

#include "kernels.h"

namespace gpt2 {

namespace {

__global__ __launch_bounds__(256) void rope_table_kernel(float2* tab, int P, int hs, double base) {
    const int half = hs / 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)P * half) return;
    const int m = (int)(idx / half), i = (int)(idx % half);
    const double a = (double)m * pow(base, -2.0 * i / hs);
    tab[idx] = make_float2((float)cos(a), (float)sin(a));
}

// Thread: one 16-byte chunk (KV values, KV / 2 pairs) of the first ncols columns of a
// row; the chunk lies inside one head (hs % KV == 0).  Row r is at position
// pos0 + r % period.  sgn = -1 turns back (the transpose).
template <class T>
__global__ __launch_bounds__(256) void rope_kernel(T* x, int64_t ld, int rows, int ncols, int hs, int period, int pos0,
                                                   const float2* __restrict__ tab, float sgn) {
    constexpr int KV = Vec16<T>::N;
    const int cpr = ncols / KV;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)rows * cpr) return;
    const int r = (int)(idx / cpr), c0 = (int)(idx % cpr) * KV;
    const int m = pos0 + r % period;
    const float2* tr = tab + (int64_t)m * (hs / 2) + (c0 % hs) / 2;
    T* p = x + (int64_t)r * ld + c0;
    float v[KV];
    unpack16<T>(ld16(p), v);
#pragma unroll
    for (int j = 0; j < KV / 2; ++j) {
        const float2 cs = tr[j];
        const float s = sgn * cs.y, x0 = v[2 * j], x1 = v[2 * j + 1];
        v[2 * j] = x0 * cs.x - x1 * s;
        v[2 * j + 1] = x0 * s + x1 * cs.x;
    }
    st16(p, pack16<T>(v));
}

}  // namespace

hipError_t rope_table(float2* tab, int P, int hs, double base, hipStream_t s) {
    if (P <= 0 || hs <= 0 || hs % 2 || !(base > 1.0)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)(((int64_t)P * (hs / 2) + 255) / 256)), dim3(256), 0, s, tab,
                       P, hs, base);
    return hipGetLastError();
}

template <class T>
hipError_t rope_apply(T* x, int64_t ld, int rows, int ncols, int hs, int period, int pos0, const float2* tab,
                      bool inverse, hipStream_t s) {
    constexpr int KV = Vec16<T>::N;
    if (rows <= 0) return hipSuccess;
    if (hs % KV || ncols % hs || ld % KV || period <= 0 || pos0 < 0) return hipErrorInvalidValue;
    // algorithmic bytes: the q | k columns read and written once, and the table rows of
    // the positions present (read once; the rows are reused across sequences)
    const double table = (double)std::min(period, rows) * (hs / 2) * 8;
    ProfScope prof(s, inverse ? "rope_bwd" : "rope_fwd", 0, 2.0 * rows * ncols * sizeof(T) + table);
    const int64_t threads = (int64_t)rows * (ncols / KV);
    hipLaunchKernelGGL(rope_kernel<T>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, x, ld, rows, ncols, hs,
                       period, pos0, tab, inverse ? -1.f : 1.f);
    return hipGetLastError();
}

template hipError_t rope_apply<float>(float*, int64_t, int, int, int, int, int, const float2*, bool, hipStream_t);
template hipError_t rope_apply<bf16>(bf16*, int64_t, int, int, int, int, int, const float2*, bool, hipStream_t);

}  // namespace gpt2
