// Exclusive prefix sum of int32 counts into int64 offsets (used by the CSR
// build and the long-row schedule).  Three passes: per-block totals, a scan
// of the block totals by one workgroup, then per-block scans plus offsets.
#include "common.h"

namespace sag {
namespace {

constexpr int kThreads = 1024;
constexpr int kPerThread = 4;
constexpr int kChunk = kThreads * kPerThread;

// Inclusive scan of one int64 per thread across a 1024-thread block.
__device__ int64_t block_inclusive_scan(int64_t v, int64_t* lds_wave /*[16]*/) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int64_t t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    if (lane == 63) lds_wave[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int64_t w = lane < kThreads / 64 ? lds_wave[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            int64_t t = __shfl_up(w, o, 64);
            if (lane >= o) w += t;
        }
        if (lane < kThreads / 64) lds_wave[lane] = w;
    }
    __syncthreads();
    if (wave > 0) v += lds_wave[wave - 1];
    __syncthreads();
    return v;
}

__global__ __launch_bounds__(kThreads) void block_totals(const int32_t* __restrict__ in, int64_t n,
                                                        int64_t* __restrict__ totals) {
    __shared__ int64_t lw[16];
    int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk + threadIdx.x * kPerThread;
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
        if (base + i < n) s += in[base + i];
    s = block_inclusive_scan(s, lw);
    if (threadIdx.x == kThreads - 1) totals[blockIdx.x] = s;
}

// One workgroup: exclusive scan of nb totals in place; total -> *grand.
__global__ __launch_bounds__(kThreads) void scan_totals(int64_t* __restrict__ totals, int64_t nb,
                                                       int64_t* __restrict__ grand) {
    __shared__ int64_t lw[16];
    int64_t carry = 0;
    for (int64_t b0 = 0; b0 < nb; b0 += kChunk) {
        int64_t base = b0 + threadIdx.x * kPerThread;
        int64_t v[kPerThread];
        int64_t s = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            v[i] = base + i < nb ? totals[base + i] : 0;
            s += v[i];
        }
        int64_t incl = block_inclusive_scan(s, lw);
        int64_t run = carry + incl - s;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            if (base + i < nb) totals[base + i] = run;
            run += v[i];
        }
        __shared__ int64_t last;
        if (threadIdx.x == kThreads - 1) last = incl;
        __syncthreads();
        carry += last;
        __syncthreads();
    }
    if (threadIdx.x == 0) *grand = carry;
}

__global__ __launch_bounds__(kThreads) void scan_blocks(const int32_t* __restrict__ in, int64_t n,
                                                       const int64_t* __restrict__ offs,
                                                       int64_t* __restrict__ out) {
    __shared__ int64_t lw[16];
    int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk + threadIdx.x * kPerThread;
    int64_t v[kPerThread];
    int64_t s = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        v[i] = base + i < n ? in[base + i] : 0;
        s += v[i];
    }
    int64_t run = block_inclusive_scan(s, lw) - s + offs[blockIdx.x];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        if (base + i < n) out[base + i] = run;
        run += v[i];
    }
}

}  // namespace

size_t scan_workspace_bytes(int64_t n) {
    int64_t nb = cdiv(n, kChunk);
    return static_cast<size_t>(nb + 1) * sizeof(int64_t) + 256;
}

sag_status exclusive_scan(const int32_t* in, int64_t* out, int64_t n, void* tmp, hipStream_t s) {
    int64_t nb = cdiv(n, kChunk);
    int64_t* totals = static_cast<int64_t*>(tmp);
    if (nb > 0) {
        block_totals<<<dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, s>>>(in, n, totals);
        SAG_LAUNCH_CHECK();
    }
    scan_totals<<<1, kThreads, 0, s>>>(totals, nb, out + n);
    SAG_LAUNCH_CHECK();
    if (nb > 0) {
        scan_blocks<<<dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, s>>>(in, n, totals, out);
        SAG_LAUNCH_CHECK();
    }
    return SAG_OK;
}

}  // namespace sag
