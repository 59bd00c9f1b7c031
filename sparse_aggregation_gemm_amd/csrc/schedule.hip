// Degree-binned schedule of a CSR for the SpMM.
//
// Power-law degree laws (the workloads of the pages: Reddit, Amazon,
// ogbn-products and the DistDGL-scale graph) put a few rows with thousands of
// entries next to millions of rows with a handful.  Rows are sorted (stable
// radix sort, so deterministic) by (bin, floor(log2(len))), which gives every
// wavefront rows of similar length, and split into three bins:
//   short  (len <= kShortMax): one lane group per row, several rows per wave;
//   medium (len <= seg_len):   one wavefront per row;
//   long   (len >  seg_len):   segments of seg_len entries, one wavefront
//                              each, summed afterwards in segment order.
#include "common.h"

namespace sag {

constexpr int kShortMax = 32;

namespace {

// Sort key of each row (bin, length class, row) and the bin counts; the
// counts are added per wavefront (one atomic per wavefront and counter).
__global__ void sched_keys(const int64_t* __restrict__ indptr, int64_t n, int32_t seg_len, int row_bits,
                           uint64_t* __restrict__ keys, unsigned long long* __restrict__ counts) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool valid = r < n;
    uint64_t bin = 3;
    unsigned long long segs = 0;
    if (valid) {
        const int64_t len = indptr[r + 1] - indptr[r];
        bin = len <= kShortMax ? 0 : (len <= seg_len ? 1 : 2);
        const uint64_t cls = len == 0 ? 0 : static_cast<uint64_t>(64 - __clzll(static_cast<unsigned long long>(len)));
        keys[r] = ((bin * 64 + cls) << row_bits) | static_cast<uint64_t>(r);
        if (bin == 2) segs = static_cast<unsigned long long>((len + seg_len - 1) / seg_len);
    }
    const unsigned long long m0 = __ballot(bin == 0), m1 = __ballot(bin == 1), m2 = __ballot(bin == 2);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) segs += __shfl_xor(segs, off, 64);
    if ((threadIdx.x & 63) == 0) {
        if (m0) atomicAdd(&counts[0], static_cast<unsigned long long>(__popcll(m0)));
        if (m1) atomicAdd(&counts[1], static_cast<unsigned long long>(__popcll(m1)));
        if (m2) {
            atomicAdd(&counts[2], static_cast<unsigned long long>(__popcll(m2)));
            atomicAdd(&counts[3], segs);
        }
    }
}

__global__ void sched_records(const uint64_t* __restrict__ keys, int64_t n, int row_bits,
                              const int64_t* __restrict__ indptr, int32_t* __restrict__ rec) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t r = static_cast<int64_t>(keys[i] & ((1ull << row_bits) - 1));
    const int64_t start = indptr[r];
    int4 v;
    v.x = static_cast<int32_t>(r);
    v.y = static_cast<int32_t>(indptr[r + 1] - start);
    v.z = static_cast<int32_t>(static_cast<uint64_t>(start) & 0xffffffffu);
    v.w = static_cast<int32_t>(static_cast<uint64_t>(start) >> 32);
    reinterpret_cast<int4*>(rec)[i] = v;
}

__global__ void long_counts(const int32_t* __restrict__ rec_long, int64_t n_long, int32_t seg_len,
                            int32_t* __restrict__ cnt) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j < n_long) cnt[j] = (rec_long[4 * j + 1] + seg_len - 1) / seg_len;
}

__global__ void long_segments(const int32_t* __restrict__ rec_long, int64_t n_long, int32_t seg_len,
                              const int64_t* __restrict__ first, int32_t* __restrict__ seg,
                              int32_t* __restrict__ seg0) {
    const int64_t j = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (j > n_long) return;
    seg0[j] = static_cast<int32_t>(first[j]);
    if (j == n_long) return;
    const int32_t len = rec_long[4 * j + 1];
    const uint64_t start = static_cast<uint32_t>(rec_long[4 * j + 2]) |
                           (static_cast<uint64_t>(static_cast<uint32_t>(rec_long[4 * j + 3])) << 32);
    const int32_t ns = (len + seg_len - 1) / seg_len;
    for (int32_t q = 0; q < ns; ++q) {
        const uint64_t s0 = start + static_cast<uint64_t>(q) * seg_len;
        int4 v;
        v.x = static_cast<int32_t>(j);
        v.y = static_cast<int32_t>(s0 & 0xffffffffu);
        v.z = static_cast<int32_t>(s0 >> 32);
        v.w = (q + 1 < ns) ? seg_len : len - q * seg_len;
        reinterpret_cast<int4*>(seg)[first[j] + q] = v;
    }
}

int64_t long_bound(int64_t n_rows, int64_t nnz, int32_t seg_len) {
    const int64_t a = nnz / (static_cast<int64_t>(seg_len) + 1);
    return a < n_rows ? a : n_rows;
}

}  // namespace
}  // namespace sag

using namespace sag;

extern "C" size_t sag_csr_schedule_bytes(int64_t n_rows, int64_t nnz, int32_t seg_len) {
    if (n_rows < 0 || nnz < 0 || seg_len < 64) return 0;
    const int64_t nl = long_bound(n_rows, nnz, seg_len);
    const int64_t ns = nl + nnz / seg_len;
    return static_cast<size_t>(16 * n_rows + 16 * ns + 4 * (nl + 1));
}

extern "C" size_t sag_csr_schedule_workspace_bytes(int64_t n_rows) {
    Carver c(nullptr, 0);
    const int64_t n = n_rows > 0 ? n_rows : 1;
    c.take<unsigned long long>(4);
    c.take<uint64_t>(n);
    c.take<uint64_t>(n);
    c.take<int32_t>(n);
    c.take<int64_t>(n + 1);
    const size_t t1 = radix_sort_workspace_bytes(n), t2 = scan_workspace_bytes(n);
    c.take<char>(t1 > t2 ? t1 : t2);
    return c.used();
}

extern "C" sag_status sag_csr_schedule(sag_csr* A, int32_t seg_len, void* buf, size_t buf_bytes,
                                       void* ws, size_t ws_bytes, void* stream) {
    if (!A) return fail(SAG_E_INVALID, "schedule: null CSR");
    if (seg_len < 64 || seg_len > 65536 || seg_len % 64) return fail(SAG_E_INVALID, "schedule: seg_len must be a multiple of 64 in [64, 65536]");
    if (A->n_rows < 0 || A->nnz < 0 || A->n_rows > INT32_MAX) return fail(SAG_E_INVALID, "schedule: bad sizes");
    if (A->n_rows > 0 && !A->indptr) return fail(SAG_E_INVALID, "schedule: null indptr");
    const int64_t n = A->n_rows;
    if (!buf || buf_bytes < sag_csr_schedule_bytes(n, A->nnz, seg_len)) return fail(SAG_E_WORKSPACE, "schedule: buffer too small");
    if (!ws || ws_bytes < sag_csr_schedule_workspace_bytes(n)) return fail(SAG_E_WORKSPACE, "schedule: workspace too small");
    if (!aligned16(buf)) return fail(SAG_E_ALIGN, "schedule: buffer not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver c(ws, ws_bytes);
    const int64_t nn = n > 0 ? n : 1;
    unsigned long long* counts = c.take<unsigned long long>(4);
    uint64_t* ka = c.take<uint64_t>(nn);
    uint64_t* kb = c.take<uint64_t>(nn);
    int32_t* cnt = c.take<int32_t>(nn);
    int64_t* first = c.take<int64_t>(nn + 1);
    const size_t t1 = radix_sort_workspace_bytes(nn), t2 = scan_workspace_bytes(nn);
    const size_t tb = t1 > t2 ? t1 : t2;
    void* tmp = c.take<char>(tb);

    const int row_bits = bits_for(n > 0 ? static_cast<uint64_t>(n - 1) : 0);
    SAG_CHECK_HIP(hipMemsetAsync(counts, 0, 4 * sizeof(unsigned long long), s));
    if (n > 0) {
        sched_keys<<<dim3(static_cast<unsigned>(cdiv(n, 256))), 256, 0, s>>>(A->indptr, n, seg_len, row_bits, ka, counts);
        SAG_LAUNCH_CHECK();
    }
    uint64_t* sorted = nullptr;
    SAG_TRY(radix_sort_u64(ka, kb, n, row_bits + 8, tmp, tb, s, &sorted));
    int32_t* rec = static_cast<int32_t*>(buf);
    if (n > 0) {
        sched_records<<<dim3(static_cast<unsigned>(cdiv(n, 256))), 256, 0, s>>>(sorted, n, row_bits, A->indptr, rec);
        SAG_LAUNCH_CHECK();
    }
    unsigned long long h[4] = {0, 0, 0, 0};
    SAG_CHECK_HIP(hipMemcpyAsync(h, counts, sizeof(h), hipMemcpyDeviceToHost, s));
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    const int64_t n_short = static_cast<int64_t>(h[0]), n_medium = static_cast<int64_t>(h[1]);
    const int64_t n_long = static_cast<int64_t>(h[2]), n_seg = static_cast<int64_t>(h[3]);
    int32_t* seg = rec + 4 * n;
    int32_t* seg0 = seg + 4 * n_seg;
    if (n_long > 0) {
        const int32_t* rec_long = rec + 4 * (n_short + n_medium);
        long_counts<<<dim3(static_cast<unsigned>(cdiv(n_long, 256))), 256, 0, s>>>(rec_long, n_long, seg_len, cnt);
        SAG_LAUNCH_CHECK();
        SAG_TRY(exclusive_scan(cnt, first, n_long, tmp, s));
        long_segments<<<dim3(static_cast<unsigned>(cdiv(n_long + 1, 256))), 256, 0, s>>>(rec_long, n_long, seg_len,
                                                                                        first, seg, seg0);
        SAG_LAUNCH_CHECK();
    }
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    A->sched = rec;
    A->n_short = n_short;
    A->n_medium = n_medium;
    A->n_long = n_long;
    A->n_seg = n_seg;
    A->seg_len = seg_len;
    return SAG_OK;
}
