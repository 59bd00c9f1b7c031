// Opt-in HIP-event timing of internal operations (see trace.cpp).
#pragma once

#include "common.h"

namespace sag {

bool trace_enabled();

// Records a start event on construction and a stop event on destruction when
// tracing is on; does nothing otherwise.
class TraceScope {
public:
    TraceScope(const std::string& name, hipStream_t s, int64_t bytes, int64_t flops);
    ~TraceScope();
    TraceScope(const TraceScope&) = delete;
    TraceScope& operator=(const TraceScope&) = delete;

private:
    hipStream_t stream_;
    int64_t index_;
};

std::string shape_name(const char* op, const char* dtype, int64_t a, int64_t b, int64_t c);

}  // namespace sag
