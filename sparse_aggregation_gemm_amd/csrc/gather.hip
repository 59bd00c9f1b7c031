// Halo gather and push: the DIGEST "pull", which copies the stale
// representations of the out-of-subgraph neighbours H~_out into the layer's
// input, and the "push", which stores a partition's newly computed rows of
// its own nodes into the representation store (DIGEST, system design: nodes
// are independent, so rows move in parallel at node granularity).  The push
// with accumulation is the return of halo gradients to their owners
// (Sylvie, "Backward Propagation": the feature gradients of halo nodes are
// sent back and integrated).  Bitwise row copies in 16-byte vectors: a group
// of lanes per row, several rows per workgroup; source rows are read once,
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

// dst[ids[k] - row_base] = src[k] (or += in fp32 with one rounding); rows
// whose target lies outside [0, n_dst) are skipped.
template <int kLanes, class T, bool ACC>
__global__ __launch_bounds__(256) void push_rows(const char* __restrict__ src, int64_t pitch_src,
                                                 const int32_t* __restrict__ ids, int64_t row_base, int64_t n,
                                                 int64_t d, int64_t n_dst, char* __restrict__ dst,
                                                 int64_t pitch_dst) {
    constexpr int kRowsPerBlock = 256 / kLanes;
    constexpr int V = Vec<T>::N;
    const int sub = threadIdx.x % kLanes;
    const int64_t k = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + threadIdx.x / kLanes;
    if (k >= n) return;
    const int64_t t = static_cast<int64_t>(ids[k]) - row_base;
    if (t < 0 || t >= n_dst) return;
    const T* s = reinterpret_cast<const T*>(src + k * pitch_src);
    T* o = reinterpret_cast<T*>(dst + t * pitch_dst);
    for (int64_t c = sub; c * V < d; c += kLanes) {
        const int64_t c0 = c * V;
        const int m = static_cast<int>(d - c0 < V ? d - c0 : V);
        if (m == V) {
            const uint4 v = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + c0)));
            if constexpr (ACC) {
                float a[V], b[V];
                unpack<T>(v, a);
                unpack<T>(*reinterpret_cast<const uint4*>(o + c0), b);
#pragma unroll
                for (int e = 0; e < V; ++e) b[e] += a[e];
                store_vals<T>(o + c0, b, V);
            } else {
                *reinterpret_cast<uint4*>(o + c0) = v;
            }
        } else {
            for (int e = 0; e < m; ++e) {
                if constexpr (ACC) o[c0 + e] = from_f32<T>(to_f32(o[c0 + e]) + to_f32(s[c0 + e]));
                else o[c0 + e] = s[c0 + e];
            }
        }
    }
}

template <int kLanes, class T, bool ACC>
sag_status launch_push(const void* src, int64_t pitch_src, const int32_t* ids, int64_t row_base, int64_t n,
                       int64_t d, int64_t n_dst, void* dst, int64_t pitch_dst, hipStream_t s) {
    constexpr int kRowsPerBlock = 256 / kLanes;
    push_rows<kLanes, T, ACC><<<dim3(static_cast<unsigned>(cdiv(n, kRowsPerBlock))), dim3(256), 0, s>>>(
        static_cast<const char*>(src), pitch_src, ids, row_base, n, d, n_dst, static_cast<char*>(dst), pitch_dst);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

template <class T, bool ACC>
sag_status push_typed(const void* src, int64_t pitch_src, const int32_t* ids, int64_t row_base, int64_t n,
                      int64_t d, int64_t n_dst, void* dst, int64_t pitch_dst, hipStream_t s) {
    const int64_t vecs = cdiv(d, Vec<T>::N);
    if (vecs <= 4) return launch_push<4, T, ACC>(src, pitch_src, ids, row_base, n, d, n_dst, dst, pitch_dst, s);
    if (vecs <= 8) return launch_push<8, T, ACC>(src, pitch_src, ids, row_base, n, d, n_dst, dst, pitch_dst, s);
    if (vecs <= 16) return launch_push<16, T, ACC>(src, pitch_src, ids, row_base, n, d, n_dst, dst, pitch_dst, s);
    if (vecs <= 32) return launch_push<32, T, ACC>(src, pitch_src, ids, row_base, n, d, n_dst, dst, pitch_dst, s);
    return launch_push<64, T, ACC>(src, pitch_src, ids, row_base, n, d, n_dst, dst, pitch_dst, s);
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

extern "C" sag_status sag_halo_push(const void* src, int64_t ld_src, const int32_t* ids, int64_t row_base,
                                    int64_t n, int64_t d, sag_dtype dt, int accumulate, void* dst,
                                    int64_t ld_dst, int64_t n_dst, void* stream) {
    using namespace sag;
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "halo_push: bad dtype");
    if (n < 0 || d < 0 || n_dst < 0) return fail(SAG_E_INVALID, "halo_push: negative size");
    if (n == 0 || d == 0 || n_dst == 0) return SAG_OK;
    if (!ids) return fail(SAG_E_INVALID, "halo_push: null ids");
    SAG_TRY(check_dense("halo_push src", src, n, d, ld_src, dt));
    SAG_TRY(check_dense("halo_push dst", dst, n_dst, d, ld_dst, dt));
    const int64_t e = elt_size(dt);
    hipStream_t s = static_cast<hipStream_t>(stream);
    TraceScope trace(trace_enabled() ? shape_name("halo_push", dt == SAG_BF16 ? "bf16" : "f32", n, d, accumulate)
                                     : std::string(),
                     s, n * ((accumulate ? 3 : 2) * d * e + 4), accumulate ? n * d : 0);
    if (dt == SAG_BF16)
        return accumulate ? push_typed<uint16_t, true>(src, ld_src * e, ids, row_base, n, d, n_dst, dst, ld_dst * e, s)
                          : push_typed<uint16_t, false>(src, ld_src * e, ids, row_base, n, d, n_dst, dst, ld_dst * e, s);
    return accumulate ? push_typed<float, true>(src, ld_src * e, ids, row_base, n, d, n_dst, dst, ld_dst * e, s)
                      : push_typed<float, false>(src, ld_src * e, ids, row_base, n, d, n_dst, dst, ld_dst * e, s);
}
