// Process-wide launch profiler: when enabled, a pair of HIP events is recorded on
// the launching stream around every kernel launch of the library, tagged with
// the kernel's name and its algorithmic flops and bytes.  Reading aggregates the
// elapsed times per name.  Recording stops silently after kMaxRecords launches.
#include <string.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "kernels.h"

namespace gpt2 {
namespace {

constexpr size_t kMaxRecords = 32768;

struct Rec {
    const char* name;
    hipEvent_t a, b;
    double flops, bytes;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;  // events are reused across enable cycles
size_t g_pool_used = 0;
int64_t g_dropped = 0;

hipEvent_t take_event() {
    if (g_pool_used == g_pool.size()) {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        g_pool.push_back(e);
    }
    return g_pool[g_pool_used++];
}

}  // namespace

bool profiling() { return g_on; }

ProfScope::ProfScope(hipStream_t s, const char* name, double flops, double bytes) : idx(-1), stream(s) {
    if (!g_on) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    if (g_recs.size() >= kMaxRecords) {
        ++g_dropped;
        return;
    }
    hipEvent_t a = take_event(), b = take_event();
    if (!a || !b) return;
    hipEventRecord(a, s);
    g_recs.push_back(Rec{name, a, b, flops, bytes});
    idx = (int)g_recs.size() - 1;
}

ProfScope::~ProfScope() {
    if (idx < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (idx < (int)g_recs.size()) hipEventRecord(g_recs[idx].b, stream);
}

}  // namespace gpt2

extern "C" {

int gpt2_profile(int enable) {
    std::lock_guard<std::mutex> lk(gpt2::g_mu);
    if (enable) {
        gpt2::g_recs.clear();
        gpt2::g_pool_used = 0;
        gpt2::g_dropped = 0;
    }
    gpt2::g_on = enable != 0;
    return GPT2_OK;
}

int gpt2_profile_read(gpt2_kernel_stat* out, int32_t max_entries, int32_t* n_entries) {
    std::lock_guard<std::mutex> lk(gpt2::g_mu);
    std::map<std::string, gpt2_kernel_stat> agg;
    for (const auto& r : gpt2::g_recs) {
        if (hipEventSynchronize(r.b) != hipSuccess) return GPT2_E_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return GPT2_E_HIP;
        gpt2_kernel_stat& s = agg[r.name];
        if (s.launches == 0) {
            strncpy(s.name, r.name, sizeof(s.name) - 1);
            s.name[sizeof(s.name) - 1] = 0;
        }
        s.launches += 1;
        s.total_ms += ms;
        s.flops += r.flops;
        s.bytes += r.bytes;
    }
    int n = 0;
    for (auto& kv : agg) {
        if (out && n < max_entries) out[n] = kv.second;
        ++n;
    }
    if (n_entries) *n_entries = n;
    return GPT2_OK;
}

int gpt2_profile_order(int32_t* out, int32_t max_entries, int32_t* n_entries) {
    std::lock_guard<std::mutex> lk(gpt2::g_mu);
    std::map<std::string, int32_t> rank;
    for (const auto& r : gpt2::g_recs) rank.emplace(r.name, 0);
    int32_t k = 0;
    for (auto& kv : rank) kv.second = k++;
    int32_t n = 0;
    for (const auto& r : gpt2::g_recs) {
        if (out && n < max_entries) out[n] = rank[r.name];
        ++n;
    }
    if (n_entries) *n_entries = n;
    return GPT2_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- matrix-core rate probe
// Every wave runs `iters` rounds of NCH independent MFMA chains on register operands
// (no memory traffic), so the launch measures the sustained issue rate of one MFMA
// form over the whole chip at the clock it holds under that load.  The accumulators
// are stored only when `sink` is non-null and the flag is set, which the compiler
// cannot know, so the chains are not removed.
namespace gpt2 {
namespace {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef float f32x16_p __attribute__((ext_vector_type(16)));
typedef float f32x4_p __attribute__((ext_vector_type(4)));
typedef int i32x8_p __attribute__((ext_vector_type(8)));

constexpr int NCH = 4;

// Operand bits that look like trained-model data (mixed signs, full mantissas): the
// matrix cores draw more power on such data than on small integers or zeros, and the
// clock they hold under load follows.
__device__ __forceinline__ uint32_t probe_bits(int lane, int e) {
    uint32_t h = (uint32_t)(lane * 8 + e) * 2654435761u;
    h ^= h >> 15;
    h *= 2246822519u;
    h ^= h >> 13;
    // E4M3 bytes / bf16 halves with exponents near 1: keep sign and mantissa bits random
    return (h & 0x87878787u) | 0x30303030u;
}
__device__ __forceinline__ float probe_value(int lane, int e) {
    const uint32_t h = probe_bits(lane, e);
    return ((float)(h & 0xffffu) / 65536.0f - 0.5f) * 0.125f;
}

template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int iters, float* sink, int store) {
    const int lane = threadIdx.x & 63;
    if constexpr (KIND == 0 || KIND == 2) {
        f32x16_p acc[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        if constexpr (KIND == 0) {
            bf16x8_p a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (__bf16)probe_value(lane, e), b[e] = (__bf16)probe_value(lane + 64, e);
            for (int i = 0; i < iters; ++i)
#pragma unroll
                for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        } else {
            i32x8_p a, b;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = (int)probe_bits(lane, e), b[e] = (int)probe_bits(lane + 64, e);
            for (int i = 0; i < iters; ++i)
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
        }
        if (store && sink) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 16; ++e) s += acc[c][e];
            sink[blockIdx.x * 256 + threadIdx.x] = s;
        }
    } else {
        f32x4_p acc[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[c][e] = 0.f;
        bf16x8_p a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (__bf16)probe_value(lane, e), b[e] = (__bf16)probe_value(lane + 64, e);
        for (int i = 0; i < iters; ++i)
#pragma unroll
            for (int c = 0; c < NCH; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
        if (store && sink) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) s += acc[c][e];
            sink[blockIdx.x * 256 + threadIdx.x] = s;
        }
    }
}

}  // namespace
}  // namespace gpt2

extern "C" {

int gpt2_mfma_peak(int32_t kind, double* tflops, void* stream) {
    using namespace gpt2;
    if (!tflops) return report_error(GPT2_E_INVAL, "tflops is NULL");
    if (kind < 0 || kind > 2) return report_error(GPT2_E_INVAL, "kind must be 0 (bf16 32x32x16), 1 (bf16 16x16x32) or 2 (MX fp8 32x32x64)");
    hipStream_t s = (hipStream_t)stream;
    // 2 blocks of 4 waves per CU (256 CUs): two waves per SIMD, each with NCH
    // independent chains (more waves per SIMD only add issue contention)
    const int blocks = 512, iters = kind == 2 ? 4096 : 8192;
    const double flops_per_mfma = kind == 0 ? 32768.0 : kind == 1 ? 16384.0 : 131072.0;
    const double flops = flops_per_mfma * NCH * iters * (blocks * 4.0);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return report_error(GPT2_E_HIP, "hipEventCreate");
    if (hipEventCreate(&e1) != hipSuccess) {
        hipEventDestroy(e0);
        return report_error(GPT2_E_HIP, "hipEventCreate");
    }
    double best = 0.0;
    int rc = GPT2_OK;
    for (int rep = 0; rep < 4 && rc == GPT2_OK; ++rep) {  // the first launch warms the clock up
        hipEventRecord(e0, s);
        if (kind == 0) hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(blocks), dim3(256), 0, s, iters, (float*)nullptr, 0);
        else if (kind == 1) hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(blocks), dim3(256), 0, s, iters, (float*)nullptr, 0);
        else hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3(blocks), dim3(256), 0, s, iters, (float*)nullptr, 0);
        hipEventRecord(e1, s);
        float ms = 0.f;
        if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            rc = report_error(GPT2_E_HIP, "mfma probe launch failed");
            break;
        }
        if (rep > 0 && ms > 0.f) best = std::max(best, flops / (ms * 1e-3) / 1e12);
    }
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    *tflops = best;
    return rc;
}

}  // extern "C"
