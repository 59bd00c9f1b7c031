// Stable least-significant-digit radix sort of uint64 keys (8 bits per
// pass), used by the CSR build (row-major entry order, the transposed
// matrix) and by the degree-binned schedule.  Each pass: per-tile digit
// histograms stored digit-major, one exclusive scan over them, and a stable
// scatter in which every wavefront ranks equal digits with ballots.
// Integer-only, so the output never depends on thread timing.
#include "common.h"

namespace sag {
namespace {

constexpr int kThreads = 256;
constexpr int kRounds = 16;                 // keys per thread per tile
constexpr int kTile = kThreads * kRounds;   // 4096 keys per workgroup
constexpr int kDigits = 256;

__global__ __launch_bounds__(kThreads) void rs_hist(const uint64_t* __restrict__ keys, int64_t n,
                                                    int shift, int32_t* __restrict__ hist,
                                                    int64_t n_tiles) {
    __shared__ int32_t cnt[kDigits];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
#pragma unroll 4
    for (int r = 0; r < kRounds; ++r) {
        int64_t i = base + r * kThreads + threadIdx.x;
        if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & 0xff], 1);
    }
    __syncthreads();
    hist[static_cast<int64_t>(threadIdx.x) * n_tiles + blockIdx.x] = cnt[threadIdx.x];
}

__global__ __launch_bounds__(kThreads) void rs_scatter(const uint64_t* __restrict__ keys, int64_t n,
                                                       int shift, const int64_t* __restrict__ offs,
                                                       int64_t n_tiles, uint64_t* __restrict__ out) {
    __shared__ int64_t base_off[kDigits];
    __shared__ int32_t wcnt[kThreads / 64][kDigits];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    base_off[threadIdx.x] = offs[static_cast<int64_t>(threadIdx.x) * n_tiles + blockIdx.x];
    for (int w = 0; w < kThreads / 64; ++w) wcnt[w][threadIdx.x] = 0;
    __syncthreads();
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTile;
    for (int r = 0; r < kRounds; ++r) {
        const int64_t i = base + r * kThreads + threadIdx.x;
        const bool valid = i < n;
        const uint64_t key = valid ? keys[i] : 0ull;
        const uint32_t digit = static_cast<uint32_t>((key >> shift) & 0xff);
        // lanes of this wavefront holding a valid key with the same digit
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (digit >> b) & 1u;
            const uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        const int rank = __popcll(peers & lt_mask);
        if (valid && rank == 0) wcnt[wave][digit] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int64_t pos = base_off[digit] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][digit];
            out[pos] = key;
        }
        __syncthreads();
        int32_t tot = 0;
        for (int w = 0; w < kThreads / 64; ++w) {
            tot += wcnt[w][threadIdx.x];
            wcnt[w][threadIdx.x] = 0;
        }
        base_off[threadIdx.x] += tot;
        __syncthreads();
    }
}

// indptr[r] = first entry whose row is >= r.
__global__ void rows_kernel(const uint64_t* __restrict__ keys, int64_t n, uint64_t divisor,
                            int64_t n_rows, int64_t* __restrict__ indptr) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t r = static_cast<int64_t>(keys[i] / divisor);
    const int64_t r_prev = i == 0 ? -1 : static_cast<int64_t>(keys[i - 1] / divisor);
    for (int64_t q = r_prev + 1; q <= r; ++q) indptr[q] = i;
    if (i == n - 1)
        for (int64_t q = r + 1; q <= n_rows; ++q) indptr[q] = n;
}

__global__ void fill_i64(int64_t* __restrict__ p, int64_t n, int64_t v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace

size_t radix_sort_workspace_bytes(int64_t n) {
    const int64_t tiles = cdiv(n, kTile);
    const int64_t cells = tiles * kDigits;
    Carver c(nullptr, 0);
    c.take<int32_t>(cells);
    c.take<int64_t>(cells + 1);
    c.take<char>(scan_workspace_bytes(cells));
    return c.used();
}

sag_status radix_sort_u64(uint64_t* keys, uint64_t* alt, int64_t n, int bits, void* tmp,
                          size_t tmp_bytes, hipStream_t s, uint64_t** result) {
    *result = keys;
    if (n <= 1 || bits <= 0) return SAG_OK;
    if (tmp_bytes < radix_sort_workspace_bytes(n))
        return fail(SAG_E_WORKSPACE, "radix sort: temporary buffer too small");
    const int64_t tiles = cdiv(n, kTile);
    const int64_t cells = tiles * kDigits;
    Carver c(tmp, tmp_bytes);
    int32_t* hist = c.take<int32_t>(cells);
    int64_t* offs = c.take<int64_t>(cells + 1);
    void* scan_tmp = c.take<char>(scan_workspace_bytes(cells));
    uint64_t* src = keys;
    uint64_t* dst = alt;
    for (int shift = 0; shift < bits; shift += 8) {
        rs_hist<<<dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s>>>(src, n, shift, hist, tiles);
        SAG_LAUNCH_CHECK();
        SAG_TRY(exclusive_scan(hist, offs, cells, scan_tmp, s));
        rs_scatter<<<dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s>>>(src, n, shift, offs, tiles, dst);
        SAG_LAUNCH_CHECK();
        uint64_t* t = src;
        src = dst;
        dst = t;
    }
    *result = src;
    return SAG_OK;
}

sag_status rows_from_sorted_keys(const uint64_t* keys, int64_t n, uint64_t divisor,
                                 int64_t n_rows, int64_t* indptr, hipStream_t s) {
    if (n == 0) {
        fill_i64<<<dim3(static_cast<unsigned>(cdiv(n_rows + 1, 256))), dim3(256), 0, s>>>(indptr, n_rows + 1, 0);
        SAG_LAUNCH_CHECK();
        return SAG_OK;
    }
    rows_kernel<<<dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, s>>>(keys, n, divisor, n_rows, indptr);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace sag
