// Opt-in measurement: HIP events recorded on the caller's stream around each
// internal operation (SpMM, dense products, gather, mask, build), with the
// operation's algorithmic bytes and flops.  Process-wide state guarded by a
// mutex; off unless sag_trace_enable(1) was called.
#include <cstdio>
#include <mutex>
#include <vector>

#include "trace.h"

namespace sag {
namespace {

struct Rec {
    std::string name;
    hipEvent_t a = nullptr, b = nullptr;
    int64_t bytes = 0, flops = 0;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;

}  // namespace

bool trace_enabled() {
    std::lock_guard<std::mutex> l(g_mu);
    return g_on;
}

TraceScope::TraceScope(const std::string& name, hipStream_t s, int64_t bytes, int64_t flops)
    : stream_(s), index_(-1) {
    std::lock_guard<std::mutex> l(g_mu);
    if (!g_on) return;
    Rec r;
    r.name = name;
    r.bytes = bytes;
    r.flops = flops;
    if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
    if (hipEventRecord(r.a, s) != hipSuccess) return;
    g_recs.push_back(r);
    index_ = static_cast<int64_t>(g_recs.size()) - 1;
}

TraceScope::~TraceScope() {
    if (index_ < 0) return;
    std::lock_guard<std::mutex> l(g_mu);
    if (index_ < static_cast<int64_t>(g_recs.size())) (void)hipEventRecord(g_recs[index_].b, stream_);
}

std::string shape_name(const char* op, const char* dtype, int64_t a, int64_t b, int64_t c) {
    char buf[160];
    std::snprintf(buf, sizeof(buf), "%s[%s,%lld,%lld,%lld]", op, dtype, static_cast<long long>(a),
                  static_cast<long long>(b), static_cast<long long>(c));
    return buf;
}

}  // namespace sag

using namespace sag;

extern "C" sag_status sag_trace_enable(int on) {
    std::lock_guard<std::mutex> l(g_mu);
    g_on = on != 0;
    return SAG_OK;
}

extern "C" int64_t sag_trace_count(void) {
    std::lock_guard<std::mutex> l(g_mu);
    return static_cast<int64_t>(g_recs.size());
}

extern "C" sag_status sag_trace_get(int64_t i, char* name, size_t name_cap, float* ms, int64_t* bytes,
                                    int64_t* flops) {
    Rec r;
    {
        std::lock_guard<std::mutex> l(g_mu);
        if (i < 0 || i >= static_cast<int64_t>(g_recs.size())) return fail(SAG_E_INVALID, "trace: index out of range");
        r = g_recs[i];
    }
    if (name && name_cap) {
        std::snprintf(name, name_cap, "%s", r.name.c_str());
    }
    if (bytes) *bytes = r.bytes;
    if (flops) *flops = r.flops;
    if (ms) {
        SAG_CHECK_HIP(hipEventSynchronize(r.b));
        SAG_CHECK_HIP(hipEventElapsedTime(ms, r.a, r.b));
    }
    return SAG_OK;
}

extern "C" sag_status sag_trace_clear(void) {
    std::lock_guard<std::mutex> l(g_mu);
    for (Rec& r : g_recs) {
        if (r.b) (void)hipEventSynchronize(r.b);
        if (r.a) (void)hipEventDestroy(r.a);
        if (r.b) (void)hipEventDestroy(r.b);
    }
    g_recs.clear();
    return SAG_OK;
}
