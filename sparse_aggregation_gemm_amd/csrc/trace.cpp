// Opt-in measurement: HIP events recorded on the caller's stream around each
// internal operation (SpMM, dense products, gather, mask, build), with the
// operation's algorithmic bytes and flops.  The switch and the records are
// per host thread (thread_local), so concurrent callers neither see nor
// disturb each other's records; off unless the thread called
// sag_trace_enable(1).  No computation reads this state.
#include <cstdio>
#include <vector>

#include "trace.h"

namespace sag {
namespace {

struct Rec {
    std::string name;
    hipEvent_t a = nullptr, b = nullptr;
    int64_t bytes = 0, flops = 0;
};

thread_local bool t_on = false;
thread_local std::vector<Rec> t_recs;

}  // namespace

bool trace_enabled() { return t_on; }

TraceScope::TraceScope(const std::string& name, hipStream_t s, int64_t bytes, int64_t flops)
    : stream_(s), index_(-1) {
    if (!t_on) return;
    Rec r;
    r.name = name;
    r.bytes = bytes;
    r.flops = flops;
    if (hipEventCreate(&r.a) != hipSuccess) return;
    if (hipEventCreate(&r.b) != hipSuccess) {
        (void)hipEventDestroy(r.a);
        return;
    }
    if (hipEventRecord(r.a, s) != hipSuccess) {
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
        return;
    }
    t_recs.push_back(r);
    index_ = static_cast<int64_t>(t_recs.size()) - 1;
}

TraceScope::~TraceScope() {
    if (index_ < 0) return;
    if (index_ < static_cast<int64_t>(t_recs.size())) (void)hipEventRecord(t_recs[index_].b, stream_);
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
    t_on = on != 0;
    return SAG_OK;
}

extern "C" int64_t sag_trace_count(void) { return static_cast<int64_t>(t_recs.size()); }

extern "C" sag_status sag_trace_get(int64_t i, char* name, size_t name_cap, float* ms, int64_t* bytes,
                                    int64_t* flops) {
    if (i < 0 || i >= static_cast<int64_t>(t_recs.size())) return fail(SAG_E_INVALID, "trace: index out of range");
    const Rec& r = t_recs[i];
    if (name && name_cap) std::snprintf(name, name_cap, "%s", r.name.c_str());
    if (bytes) *bytes = r.bytes;
    if (flops) *flops = r.flops;
    if (ms) {
        SAG_CHECK_HIP(hipEventSynchronize(r.b));
        SAG_CHECK_HIP(hipEventElapsedTime(ms, r.a, r.b));
    }
    return SAG_OK;
}

extern "C" sag_status sag_trace_clear(void) {
    for (Rec& r : t_recs) {
        if (r.b) (void)hipEventSynchronize(r.b);
        if (r.a) (void)hipEventDestroy(r.a);
        if (r.b) (void)hipEventDestroy(r.b);
    }
    t_recs.clear();
    return SAG_OK;
}
