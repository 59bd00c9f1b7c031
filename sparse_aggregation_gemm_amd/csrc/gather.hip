// Halo gather: the DIGEST "pull", which copies the stale representations of
// the out-of-subgraph neighbours H~_out into the layer's input (DIGEST,
// system design: nodes are independent, so rows are copied in parallel at
// node granularity).  A bitwise row copy in 16-byte vectors: a group of
// lanes per row, several rows per workgroup; the source rows are read once,
// so the loads bypass the caches (nontemporal).
#include "common.h"
#include "trace.h"

namespace sag {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int kLanes>
__global__ __launch_bounds__(256) void gather_rows(const char* __restrict__ src, int64_t pitch_src,
                                                   const int32_t* __restrict__ rows, int64_t row_base,
                                                   int64_t n,
                                                   int64_t row_bytes, char* __restrict__ dst,
                                                   int64_t pitch_dst) {
    constexpr int kRowsPerBlock = 256 / kLanes;
    const int sub = threadIdx.x % kLanes;
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kLanes;
    if (k >= n) return;
    const char* s = src + (static_cast<int64_t>(rows[k]) - row_base) * pitch_src;
    char* d = dst + k * pitch_dst;
    const int64_t full = row_bytes / 16;
    for (int64_t c = sub; c < full; c += kLanes) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s) + c);
        *reinterpret_cast<u32x4*>(d + c * 16) = v;
    }
    // a row width that is not a multiple of 16 bytes ends in 2-byte units
    const int64_t tail = row_bytes - full * 16;
    for (int64_t b = sub * 2; b < tail; b += 2 * kLanes)
        *reinterpret_cast<uint16_t*>(d + full * 16 + b) = *reinterpret_cast<const uint16_t*>(s + full * 16 + b);
}

template <int kLanes>
sag_status launch(const void* src, int64_t pitch_src, const int32_t* rows, int64_t row_base, int64_t n,
                  int64_t row_bytes,
                  void* dst, int64_t pitch_dst, hipStream_t s) {
    constexpr int kRowsPerBlock = 256 / kLanes;
    const int64_t blocks = cdiv(n, kRowsPerBlock);
    gather_rows<kLanes><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(
        static_cast<const char*>(src), pitch_src, rows, row_base, n, row_bytes, static_cast<char*>(dst), pitch_dst);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace
}  // namespace sag

extern "C" sag_status sag_halo_gather(const void* src, int64_t ld_src, const int32_t* rows, int64_t row_base,
                                      int64_t n, int64_t d, sag_dtype dt, void* dst, int64_t ld_dst,
                                      void* stream) {
    using namespace sag;
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "halo_gather: bad dtype");
    if (n < 0 || d < 0) return fail(SAG_E_INVALID, "halo_gather: negative size");
    if (n == 0 || d == 0) return SAG_OK;
    if (!rows) return fail(SAG_E_INVALID, "halo_gather: null rows");
    SAG_TRY(check_dense("halo_gather src", src, 1, d, ld_src, dt));
    SAG_TRY(check_dense("halo_gather dst", dst, n, d, ld_dst, dt));
    const int64_t e = elt_size(dt);
    const int64_t row_bytes = d * e;
    const int64_t chunks = cdiv(row_bytes, 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    TraceScope trace(trace_enabled() ? shape_name("halo_gather", dt == SAG_BF16 ? "bf16" : "f32", n, d, 0) : std::string(),
                     s, n * (2 * row_bytes + 4), 0);
    if (chunks <= 4) return launch<4>(src, ld_src * e, rows, row_base, n, row_bytes, dst, ld_dst * e, s);
    if (chunks <= 8) return launch<8>(src, ld_src * e, rows, row_base, n, row_bytes, dst, ld_dst * e, s);
    if (chunks <= 16) return launch<16>(src, ld_src * e, rows, row_base, n, row_bytes, dst, ld_dst * e, s);
    if (chunks <= 32) return launch<32>(src, ld_src * e, rows, row_base, n, row_bytes, dst, ld_dst * e, s);
    return launch<64>(src, ld_src * e, rows, row_base, n, row_bytes, dst, ld_dst * e, s);
}
