// Process-wide launch profiler: when enabled, a pair of HIP events is recorded on
// the launching stream around every kernel launch of the library, tagged with
// the kernel's name and its algorithmic flops and bytes.  Reading aggregates the
// elapsed times per name.  Recording stops silently after kMaxRecords launches.
#include <string.h>

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

}  // extern "C"
