// Hub split of a CSR: the entries that fall in the columns holding the most
// entries (the hub columns) and the rest, as two CSRs over the same rows.
//
// A product over a dense-ish graph re-reads each row of X hundreds of times
// (once per entry in its column), but the rows are spread over far more
// memory than one XCD's L2 holds, so nearly every gather misses.  On a
// power-law degree law a few columns hold a large share of the entries: a
// first pass over those entries alone touches a few megabytes of X and is
// served from L2, and the second pass over the rest fetches a smaller share
// of rows than the one-pass product did.  The split is set-up work (once per
// matrix): integer counting, a stable radix sort of the column keys and an
// order-preserving compaction, so it is deterministic.
#include "common.h"
#include "ops.h"

namespace sag {
namespace {

constexpr int kThreads = 256;

// entries per column (integer atomics: counts do not depend on order)
__global__ void split_col_counts(const int32_t* __restrict__ idx, int64_t nnz, int32_t* __restrict__ cnt) {
    const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (e < nnz) atomicAdd(&cnt[idx[e]], 1);
}

// sort key of each column: most entries first, then the lower column id
__global__ void split_keys(const int32_t* __restrict__ cnt, int64_t n_cols, int col_bits,
                           uint64_t* __restrict__ keys) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (c < n_cols)
        keys[c] = (static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(cnt[c])) << col_bits) |
                  static_cast<uint64_t>(c);
}

__global__ void split_mark(const uint64_t* __restrict__ sorted, int64_t n_hub, uint64_t col_mask,
                           uint8_t* __restrict__ hub) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < n_hub) hub[sorted[i] & col_mask] = 1;
}

// hub entries of each row (one wavefront per row)
__global__ __launch_bounds__(kThreads) void split_row_counts(const int64_t* __restrict__ indptr,
                                                             const int32_t* __restrict__ idx, int64_t n_rows,
                                                             const uint8_t* __restrict__ hub,
                                                             int32_t* __restrict__ cnt) {
    const int64_t r = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (r >= n_rows) return;
    const int64_t b = indptr[r], e = indptr[r + 1];
    int32_t c = 0;
    for (int64_t p = b + lane; p < e; p += 64) c += hub[idx[p]];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
    if (lane == 0) cnt[r] = c;
}

__global__ void split_cold_ptr(const int64_t* __restrict__ indptr, const int64_t* __restrict__ hp, int64_t n_rows,
                               int64_t* __restrict__ cp) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (r <= n_rows) cp[r] = indptr[r] - hp[r];
}

// each row's entries to its hub or cold part, in their order (one wavefront
// per row; ballots rank the entries of each 64-entry step)
__global__ __launch_bounds__(kThreads) void split_scatter(const int64_t* __restrict__ indptr,
                                                          const int32_t* __restrict__ idx,
                                                          const float* __restrict__ val, int64_t n_rows,
                                                          const uint8_t* __restrict__ hub,
                                                          const int64_t* __restrict__ hp,
                                                          const int64_t* __restrict__ cp,
                                                          int32_t* __restrict__ hi, float* __restrict__ hv,
                                                          int32_t* __restrict__ ci, float* __restrict__ cv) {
    const int64_t r = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) >> 6;
    const int lane = threadIdx.x & 63;
    if (r >= n_rows) return;
    const int64_t b = indptr[r], e = indptr[r + 1];
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int64_t h = hp[r], c = cp[r];
    for (int64_t p0 = b; p0 < e; p0 += 64) {
        const int64_t p = p0 + lane;
        const bool in = p < e;
        const int32_t col = in ? idx[p] : 0;
        const bool is_hub = in && hub[col] != 0;
        const bool is_cold = in && !is_hub;
        const uint64_t mh = __ballot(is_hub), mc = __ballot(is_cold);
        if (is_hub) {
            const int64_t q = h + __popcll(mh & below);
            hi[q] = col;
            if (val) hv[q] = val[p];
        } else if (is_cold) {
            const int64_t q = c + __popcll(mc & below);
            ci[q] = col;
            if (val) cv[q] = val[p];
        }
        h += __popcll(mh);
        c += __popcll(mc);
    }
}

unsigned blocks_for(int64_t threads) { return static_cast<unsigned>(cdiv(threads > 0 ? threads : 1, kThreads)); }

}  // namespace
}  // namespace sag

using namespace sag;

extern "C" size_t sag_csr_hub_split_workspace_bytes(int64_t n_rows, int64_t n_cols) {
    Carver c(nullptr, 0);
    const int64_t nc = n_cols > 0 ? n_cols : 1, nr = n_rows > 0 ? n_rows : 1;
    c.take<int32_t>(nc);    // entries per column
    c.take<uint64_t>(nc);   // column keys
    c.take<uint64_t>(nc);   // radix sort's second buffer
    c.take<uint8_t>(nc);    // hub flags
    c.take<int32_t>(nr);    // hub entries per row
    const size_t t1 = radix_sort_workspace_bytes(nc), t2 = scan_workspace_bytes(nr);
    c.take<char>(t1 > t2 ? t1 : t2);
    return c.used();
}

extern "C" sag_status sag_csr_hub_split(const sag_csr* A, int64_t n_hub, int64_t cap_hub, int64_t* indptr_hub,
                                        int32_t* indices_hub, float* values_hub, int64_t cap_cold,
                                        int64_t* indptr_cold, int32_t* indices_cold, float* values_cold,
                                        int64_t* nnz_hub, void* ws, size_t ws_bytes, void* stream) {
    SAG_TRY(check_csr("hub_split", A));
    if (A->hub_part || A->cold_part) return fail(SAG_E_INVALID, "hub_split: the matrix already has a split");
    if (!nnz_hub) return fail(SAG_E_INVALID, "hub_split: null nnz_hub");
    *nnz_hub = 0;
    if (n_hub < 1) return fail(SAG_E_INVALID, "hub_split: n_hub must be at least 1");
    if (cap_hub < 0 || cap_cold < 0) return fail(SAG_E_INVALID, "hub_split: negative capacity");
    if (!indptr_hub || !indptr_cold) return fail(SAG_E_INVALID, "hub_split: null row pointers");
    if (A->values && (!values_hub || !values_cold))
        return fail(SAG_E_INVALID, "hub_split: the matrix has values, so both parts need value arrays");
    if (A->row_mean && !A->values) return fail(SAG_E_INVALID, "hub_split: a row_mean matrix must store its values");
    const int64_t n = A->n_rows, nc = A->n_cols, nnz = A->nnz;
    if (!ws || ws_bytes < sag_csr_hub_split_workspace_bytes(n, nc)) return fail(SAG_E_WORKSPACE, "hub_split: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver c(ws, ws_bytes);
    const int64_t ncc = nc > 0 ? nc : 1, nr = n > 0 ? n : 1;
    int32_t* col_cnt = c.take<int32_t>(ncc);
    uint64_t* keys = c.take<uint64_t>(ncc);
    uint64_t* alt = c.take<uint64_t>(ncc);
    uint8_t* hub = c.take<uint8_t>(ncc);
    int32_t* row_cnt = c.take<int32_t>(nr);
    const size_t t1 = radix_sort_workspace_bytes(ncc), t2 = scan_workspace_bytes(nr);
    const size_t tb = t1 > t2 ? t1 : t2;
    void* tmp = c.take<char>(tb);

    SAG_CHECK_HIP(hipMemsetAsync(hub, 0, static_cast<size_t>(ncc), s));
    if (nc > 0) {
        SAG_CHECK_HIP(hipMemsetAsync(col_cnt, 0, static_cast<size_t>(nc) * sizeof(int32_t), s));
        if (nnz > 0) {
            split_col_counts<<<blocks_for(nnz), kThreads, 0, s>>>(A->indices, nnz, col_cnt);
            SAG_LAUNCH_CHECK();
        }
        const int col_bits = bits_for(static_cast<uint64_t>(nc - 1));
        split_keys<<<blocks_for(nc), kThreads, 0, s>>>(col_cnt, nc, col_bits, keys);
        SAG_LAUNCH_CHECK();
        uint64_t* sorted = nullptr;
        SAG_TRY(radix_sort_u64(keys, alt, nc, 32 + col_bits, tmp, tb, s, &sorted));
        const int64_t k = n_hub < nc ? n_hub : nc;
        const uint64_t mask = col_bits == 0 ? 0ull : (~0ull >> (64 - col_bits));
        split_mark<<<blocks_for(k), kThreads, 0, s>>>(sorted, k, mask, hub);
        SAG_LAUNCH_CHECK();
    }
    if (n > 0) {
        split_row_counts<<<blocks_for(n * 64), kThreads, 0, s>>>(A->indptr, A->indices, n, hub, row_cnt);
        SAG_LAUNCH_CHECK();
        SAG_TRY(exclusive_scan(row_cnt, indptr_hub, n, tmp, s));
        split_cold_ptr<<<blocks_for(n + 1), kThreads, 0, s>>>(A->indptr, indptr_hub, n, indptr_cold);
        SAG_LAUNCH_CHECK();
    } else {
        SAG_CHECK_HIP(hipMemsetAsync(indptr_hub, 0, sizeof(int64_t), s));
        SAG_CHECK_HIP(hipMemsetAsync(indptr_cold, 0, sizeof(int64_t), s));
    }
    int64_t h = 0;
    SAG_CHECK_HIP(hipMemcpyAsync(&h, indptr_hub + n, sizeof(int64_t), hipMemcpyDeviceToHost, s));
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    *nnz_hub = h;
    if (h > cap_hub || nnz - h > cap_cold)
        return fail(SAG_E_WORKSPACE, "hub_split: a part holds more entries than its capacity");
    if ((h > 0 && !indices_hub) || (nnz - h > 0 && !indices_cold))
        return fail(SAG_E_INVALID, "hub_split: null index array for a part with entries");
    if (n > 0 && nnz > 0) {
        split_scatter<<<blocks_for(n * 64), kThreads, 0, s>>>(A->indptr, A->indices, A->values, n, hub, indptr_hub,
                                                             indptr_cold, indices_hub, values_hub, indices_cold,
                                                             values_cold);
        SAG_LAUNCH_CHECK();
    }
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    return SAG_OK;
}
