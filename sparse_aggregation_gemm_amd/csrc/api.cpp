// Status strings, per-thread error detail and shared host-side checks.
#include <string>

#include "common.h"

namespace sag {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

sag_status fail(sag_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

sag_status check_dense(const char* name, const void* p, int64_t rows, int64_t d, int64_t ld,
                       sag_dtype t) {
    if (t != SAG_F32 && t != SAG_BF16) return fail(SAG_E_INVALID, std::string(name) + ": bad dtype");
    if (d < 0 || rows < 0) return fail(SAG_E_INVALID, std::string(name) + ": negative size");
    if (ld < d) return fail(SAG_E_INVALID, std::string(name) + ": ld < width");
    if (rows == 0 || d == 0) return SAG_OK;
    if (!p) return fail(SAG_E_INVALID, std::string(name) + ": null pointer");
    if (!aligned16(p)) return fail(SAG_E_ALIGN, std::string(name) + ": pointer not 16-B aligned");
    if ((ld * elt_size(t)) % 16) return fail(SAG_E_ALIGN, std::string(name) + ": row pitch not a multiple of 16 B");
    return SAG_OK;
}

int device_cus() {
    static const int cus = [] {
        int dev = 0, v = 0;
        return hipGetDevice(&dev) == hipSuccess &&
                       hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
                   ? v
                   : 256;
    }();
    return cus;
}

}  // namespace sag

extern "C" {

const char* sag_status_string(sag_status s) {
    switch (s) {
        case SAG_OK: return "ok";
        case SAG_E_INVALID: return "invalid argument";
        case SAG_E_ALIGN: return "misaligned pointer or leading dimension";
        case SAG_E_WORKSPACE: return "workspace too small";
        case SAG_E_RANGE: return "edge id out of range";
        case SAG_E_HIP: return "HIP runtime error";
        case SAG_E_UNSUPPORTED: return "unsupported dtype combination";
    }
    return "unknown status";
}

const char* sag_last_error(void) { return sag::g_last_error.c_str(); }

const char* sag_version(void) { return "sag 0.1 gfx950"; }

}  // extern "C"
