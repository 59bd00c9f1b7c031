// CSR build of one partition: the normalised adjacency D^-1/2 (A+I) D^-1/2
// (or the GraphSAGE mean, or plain 0/1) of the local row range, its HALO node
// list and its transpose.
//
// Follows the CAGNET page's background section (self connections, symmetric
// normalisation with the modified degrees, A and A^T kept apart), Sylvie's
// "Graph Engine" (the halo set of a partition) and DIGEST's pull (the
// out-of-subgraph neighbours are the rows fetched from the stale store).
//
// Every entry becomes one 64-bit key  row * NC + col'  with NC = n_local +
// n_global and col' = c - lo for a local column, n_local + c for a remote
// one; col' orders local columns first and remote columns by global id,
// which is the final column order.  A full radix sort of the keys puts the
// entries in row-major order and makes duplicates adjacent, so the result is
// the same whatever order the expansion kernel emitted them in.
#include <cmath>

#include "common.h"

namespace sag {
namespace {

struct BuildGeom {
    int64_t lo, hi, n_local, n_global;
    uint64_t nc;  // key divisor
};

__device__ __forceinline__ uint64_t col_code(int64_t c, const BuildGeom& g) {
    return (c >= g.lo && c < g.hi) ? static_cast<uint64_t>(c - g.lo)
                                   : static_cast<uint64_t>(g.n_local + c);
}

// Each thread takes kExpandItems edges (strided by the block size, so loads
// stay coalesced) and emits up to two keys per edge; a workgroup reserves
// room for all its keys with one atomic and writes them at block-scan
// offsets.
constexpr int kExpandItems = 8;

__global__ __launch_bounds__(256) void expand_edges(const int32_t* __restrict__ src,
                                                    const int32_t* __restrict__ dst, int64_t n_edges,
                                                    BuildGeom g, int symmetrize,
                                                    uint64_t* __restrict__ keys,
                                                    unsigned long long* __restrict__ counter,
                                                    int* __restrict__ bad) {
    __shared__ int wave_tot[4];
    __shared__ unsigned long long block_base;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t e0 = static_cast<int64_t>(blockIdx.x) * (256 * kExpandItems) + threadIdx.x;
    uint64_t key[2 * kExpandItems];
    bool em[2 * kExpandItems];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kExpandItems; ++i) {
        const int64_t e = e0 + static_cast<int64_t>(i) * 256;
        int64_t u = -1, v = -1;
        if (e < n_edges) {
            u = src[e];
            v = dst[e];
            if (u < 0 || v < 0 || u >= g.n_global || v >= g.n_global) {
                atomicOr(bad, 1);
                u = v = -1;
            }
        }
        // u -> v: row v aggregates column u
        em[2 * i] = u >= 0 && u != v && v >= g.lo && v < g.hi;
        key[2 * i] = em[2 * i] ? static_cast<uint64_t>(v - g.lo) * g.nc + col_code(u, g) : 0;
        em[2 * i + 1] = symmetrize && u >= 0 && u != v && u >= g.lo && u < g.hi;
        key[2 * i + 1] = em[2 * i + 1] ? static_cast<uint64_t>(u - g.lo) * g.nc + col_code(v, g) : 0;
        cnt += (em[2 * i] ? 1 : 0) + (em[2 * i + 1] ? 1 : 0);
    }
    // exclusive prefix of cnt over the workgroup
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off, 64);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        before += w < wave ? wave_tot[w] : 0;
        total += wave_tot[w];
    }
    if (threadIdx.x == 0) block_base = total ? atomicAdd(counter, static_cast<unsigned long long>(total)) : 0ull;
    __syncthreads();
    unsigned long long pos = block_base + static_cast<unsigned long long>(before + incl - cnt);
#pragma unroll
    for (int j = 0; j < 2 * kExpandItems; ++j)
        if (em[j]) keys[pos++] = key[j];
}

__global__ void self_loop_keys(uint64_t* __restrict__ keys, int64_t n_local, uint64_t nc) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r < n_local) keys[r] = static_cast<uint64_t>(r) * nc + static_cast<uint64_t>(r);
}

__global__ void first_flags(const uint64_t* __restrict__ k, int64_t n, int32_t* __restrict__ f) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) f[i] = (i == 0 || k[i] != k[i - 1]) ? 1 : 0;
}

__global__ void compact_unique(const uint64_t* __restrict__ k, int64_t n, const int32_t* __restrict__ f,
                               const int64_t* __restrict__ pos, uint64_t* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n && f[i]) out[pos[i]] = k[i];
}

// mark[c] = 1 for every remote global id c that appears as a column.
__global__ void mark_halo(const uint64_t* __restrict__ k, int64_t n, uint64_t nc, int64_t n_local,
                          int32_t* __restrict__ mark) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t c = static_cast<int64_t>(k[i] % nc);
    if (c >= n_local) mark[c - n_local] = 1;
}

__global__ void halo_list(const int32_t* __restrict__ mark, const int64_t* __restrict__ rank,
                          int64_t n_global, int32_t* __restrict__ halo_gid) {
    const int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (c < n_global && mark[c]) halo_gid[rank[c]] = static_cast<int32_t>(c);
}

__global__ void final_columns(const uint64_t* __restrict__ k, int64_t n, uint64_t nc, int64_t n_local,
                              const int64_t* __restrict__ rank, int32_t* __restrict__ indices) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t c = static_cast<int64_t>(k[i] % nc);
    indices[i] = static_cast<int32_t>(c < n_local ? c : n_local + rank[c - n_local]);
}

__global__ void row_degrees(const int64_t* __restrict__ indptr, int64_t n_local, int32_t* __restrict__ deg) {
    const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r < n_local) deg[r] = static_cast<int32_t>(indptr[r + 1] - indptr[r]);
}

// Halo column degrees: from the caller's global degrees, or 1 + the number
// of local entries in the column (integer atomics: the count is exact).
__global__ void halo_degrees_given(const int32_t* __restrict__ halo_gid, int64_t n_halo,
                                   const int32_t* __restrict__ deg_global, int32_t* __restrict__ deg_halo) {
    const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (k < n_halo) deg_halo[k] = deg_global[halo_gid[k]];
}
__global__ void fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}
__global__ void halo_degrees_count(const int32_t* __restrict__ indices, int64_t nnz, int64_t n_local,
                                   int32_t* __restrict__ deg) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < nnz && indices[i] >= n_local) atomicAdd(&deg[indices[i]], 1);
}

// Entry value of (row r, column c) from the degrees, in fp64 with correctly
// rounded sqrt and divide, rounded once to fp32.
__device__ __forceinline__ float entry_value(int norm, int32_t dr, int32_t dc) {
    const double a = static_cast<double>(dr < 1 ? 1 : dr);
    const double b = static_cast<double>(dc < 1 ? 1 : dc);
    if (norm == SAG_NORM_GCN) return static_cast<float>(1.0 / sqrt(a * b));
    if (norm == SAG_NORM_MEAN) return static_cast<float>(1.0 / a);
    return 1.0f;
}

__global__ void values_a(const uint64_t* __restrict__ k, int64_t n, uint64_t nc,
                         const int32_t* __restrict__ indices, const int32_t* __restrict__ deg, int norm,
                         float* __restrict__ values) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t r = static_cast<int64_t>(k[i] / nc);
    values[i] = entry_value(norm, deg[r], deg[indices[i]]);
}

// Transposed entries: key = c * n_local + r.
__global__ void transpose_keys(const uint64_t* __restrict__ k, int64_t n, uint64_t nc,
                               const int32_t* __restrict__ indices, int64_t n_local,
                               uint64_t* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t r = k[i] / nc;
    out[i] = static_cast<uint64_t>(indices[i]) * static_cast<uint64_t>(n_local) + r;
}

__global__ void transpose_fill(const uint64_t* __restrict__ kt, int64_t n, int64_t n_local,
                               const int32_t* __restrict__ deg, int norm,
                               int32_t* __restrict__ indices_t, float* __restrict__ values_t) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t c = static_cast<int64_t>(kt[i] / static_cast<uint64_t>(n_local));
    const int64_t r = static_cast<int64_t>(kt[i] % static_cast<uint64_t>(n_local));
    indices_t[i] = static_cast<int32_t>(r);
    values_t[i] = entry_value(norm, deg[r], deg[c]);
}

inline dim3 grid_for(int64_t n) { return dim3(static_cast<unsigned>(cdiv(n > 0 ? n : 1, 256))); }

struct BuildWs {
    unsigned long long* counter;
    int* bad;
    uint64_t* keys_a;
    uint64_t* keys_b;
    int32_t* flags;       // cap entries, or n_global marks
    int64_t* pos;         // cap + 1 positions, or n_global + 1 ranks
    int32_t* deg;         // n_local + n_global
    void* tmp;
    size_t tmp_bytes;
};

BuildWs carve_build(void* ws, size_t bytes, int64_t cap, int64_t n_global, int64_t n_local) {
    Carver c(ws, bytes);
    BuildWs w;
    w.counter = c.take<unsigned long long>(1);
    w.bad = c.take<int>(1);
    w.keys_a = c.take<uint64_t>(cap);
    w.keys_b = c.take<uint64_t>(cap);
    const int64_t big = cap > n_global ? cap : n_global;
    w.flags = c.take<int32_t>(big);
    w.pos = c.take<int64_t>(big + 1);
    w.deg = c.take<int32_t>(n_local + n_global);
    const size_t t1 = radix_sort_workspace_bytes(cap);
    const size_t t2 = scan_workspace_bytes(big);
    w.tmp_bytes = t1 > t2 ? t1 : t2;
    w.tmp = c.take<char>(w.tmp_bytes);
    if (!ws) w.tmp_bytes = c.used();   // measuring: total size
    return w;
}

int64_t entry_capacity(int64_t n_edges, int64_t n_local, unsigned flags) {
    return ((flags & SAG_SYMMETRIZE) ? 2 : 1) * n_edges + ((flags & SAG_SELF_LOOPS) ? n_local : 0);
}

}  // namespace
}  // namespace sag

using namespace sag;

extern "C" size_t sag_csr_build_workspace_bytes(int64_t n_edges, int64_t n_global, int64_t lo,
                                                int64_t hi, unsigned flags) {
    if (n_edges < 0 || n_global < 0 || lo < 0 || hi < lo || hi > n_global) return 0;
    const int64_t cap = entry_capacity(n_edges, hi - lo, flags);
    BuildWs w = carve_build(nullptr, 0, cap > 0 ? cap : 1, n_global, hi - lo);
    return w.tmp_bytes;
}

namespace sag {
namespace {

// Validation of the edge-list arguments shared by the build and its query.
sag_status check_build_inputs(const int32_t* src, const int32_t* dst, int64_t n_edges, int64_t n_global, int64_t lo,
                              int64_t hi, unsigned flags) {
    if (n_edges < 0 || n_global < 0) return fail(SAG_E_INVALID, "build: negative size");
    if (n_global > INT32_MAX) return fail(SAG_E_INVALID, "build: n_global exceeds int32 ids");
    if (!(0 <= lo && lo <= hi && hi <= n_global)) return fail(SAG_E_INVALID, "build: need 0 <= lo <= hi <= n_global");
    if (flags & ~static_cast<unsigned>(SAG_SYMMETRIZE | SAG_SELF_LOOPS))
        return fail(SAG_E_INVALID, "build: unknown flag");
    if (n_edges > 0 && (!src || !dst)) return fail(SAG_E_INVALID, "build: null edge list");
    return SAG_OK;
}

// The front half of the build: keys of the 0/1 pattern sorted and made
// unique, the halo set marked and ranked.  Leaves in the workspace what the
// back half reads (the unique keys, the halo ranks in w.pos, the marks in
// w.flags) and returns the sizes.  Synchronises the stream.
struct Front {
    BuildWs w;
    BuildGeom g;
    uint64_t* uniq = nullptr;
    int64_t nnz = 0, n_halo = 0;
};

sag_status build_front(const int32_t* src, const int32_t* dst, int64_t n_edges, int64_t n_global, int64_t lo,
                       int64_t hi, unsigned flags, void* ws, size_t ws_bytes, hipStream_t s, Front& f) {
    const int64_t n_local = hi - lo;
    const uint64_t nc = static_cast<uint64_t>(n_local + n_global);
    const int key_bits = bits_for(n_local > 0 ? static_cast<uint64_t>(n_local) * nc - 1 : 0);
    if (key_bits > 63) return fail(SAG_E_UNSUPPORTED, "build: key space exceeds 63 bits");
    const int64_t cap = entry_capacity(n_edges, n_local, flags);
    if (ws_bytes < sag_csr_build_workspace_bytes(n_edges, n_global, lo, hi, flags) || !ws)
        return fail(SAG_E_WORKSPACE, "build: workspace too small");
    BuildWs& w = f.w;
    w = carve_build(ws, ws_bytes, cap > 0 ? cap : 1, n_global, n_local);
    f.g = BuildGeom{lo, hi, n_local, n_global, nc};
    const BuildGeom& g = f.g;

    // 1. expand the edge list into keys; count them; detect bad ids
    SAG_CHECK_HIP(hipMemsetAsync(w.counter, 0, sizeof(unsigned long long), s));
    SAG_CHECK_HIP(hipMemsetAsync(w.bad, 0, sizeof(int), s));
    if (n_edges > 0) {
        expand_edges<<<dim3(static_cast<unsigned>(cdiv(n_edges, 256 * kExpandItems))), 256, 0, s>>>(
            src, dst, n_edges, g, (flags & SAG_SYMMETRIZE) ? 1 : 0, w.keys_a, w.counter, w.bad);
        SAG_LAUNCH_CHECK();
    }
    unsigned long long m_edges = 0;
    int bad = 0;
    SAG_CHECK_HIP(hipMemcpyAsync(&m_edges, w.counter, sizeof(m_edges), hipMemcpyDeviceToHost, s));
    SAG_CHECK_HIP(hipMemcpyAsync(&bad, w.bad, sizeof(bad), hipMemcpyDeviceToHost, s));
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    if (bad) return fail(SAG_E_RANGE, "build: an edge id lies outside [0, n_global)");
    int64_t m = static_cast<int64_t>(m_edges);
    if (flags & SAG_SELF_LOOPS) {
        if (n_local > 0) {
            self_loop_keys<<<grid_for(n_local), 256, 0, s>>>(w.keys_a + m, n_local, nc);
            SAG_LAUNCH_CHECK();
        }
        m += n_local;
    }

    // 2. sort; 3. drop duplicates
    uint64_t* sorted = nullptr;
    SAG_TRY(radix_sort_u64(w.keys_a, w.keys_b, m, key_bits, w.tmp, w.tmp_bytes, s, &sorted));
    uint64_t* uniq = sorted == w.keys_a ? w.keys_b : w.keys_a;
    int64_t nnz = 0;
    if (m > 0) {
        first_flags<<<grid_for(m), 256, 0, s>>>(sorted, m, w.flags);
        SAG_LAUNCH_CHECK();
        SAG_TRY(exclusive_scan(w.flags, w.pos, m, w.tmp, s));
        compact_unique<<<grid_for(m), 256, 0, s>>>(sorted, m, w.flags, w.pos, uniq);
        SAG_LAUNCH_CHECK();
        SAG_CHECK_HIP(hipMemcpyAsync(&nnz, w.pos + m, sizeof(nnz), hipMemcpyDeviceToHost, s));
    }

    // 4. halo set: mark remote columns, rank them by global id
    SAG_CHECK_HIP(hipMemsetAsync(w.flags, 0, sizeof(int32_t) * (n_global > 0 ? n_global : 1), s));
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    if (nnz > 0) {
        mark_halo<<<grid_for(nnz), 256, 0, s>>>(uniq, nnz, nc, n_local, w.flags);
        SAG_LAUNCH_CHECK();
    }
    int64_t n_halo = 0;
    if (n_global > 0) {
        SAG_TRY(exclusive_scan(w.flags, w.pos, n_global, w.tmp, s));
        SAG_CHECK_HIP(hipMemcpyAsync(&n_halo, w.pos + n_global, sizeof(n_halo), hipMemcpyDeviceToHost, s));
        SAG_CHECK_HIP(hipStreamSynchronize(s));
    }
    f.uniq = uniq;
    f.nnz = nnz;
    f.n_halo = n_halo;
    return SAG_OK;
}

}  // namespace
}  // namespace sag

extern "C" sag_status sag_csr_build_normalize_query(const int32_t* src, const int32_t* dst, int64_t n_edges,
                                                    int64_t n_global, int64_t lo, int64_t hi, unsigned flags,
                                                    int64_t* nnz_out, int64_t* n_halo_out, void* ws,
                                                    size_t ws_bytes, void* stream) {
    if (!nnz_out || !n_halo_out) return fail(SAG_E_INVALID, "build_query: null size outputs");
    *nnz_out = 0;
    *n_halo_out = 0;
    SAG_TRY(check_build_inputs(src, dst, n_edges, n_global, lo, hi, flags));
    Front f;
    SAG_TRY(build_front(src, dst, n_edges, n_global, lo, hi, flags, ws, ws_bytes, static_cast<hipStream_t>(stream),
                        f));
    *nnz_out = f.nnz;
    *n_halo_out = f.n_halo;
    return SAG_OK;
}

extern "C" sag_status sag_csr_build_normalize(const int32_t* src, const int32_t* dst, int64_t n_edges,
                                              int64_t n_global, int64_t lo, int64_t hi, unsigned flags,
                                              sag_norm norm, const int32_t* deg_global,
                                              int64_t cap_nnz, int64_t cap_halo,
                                              int64_t* indptr, int32_t* indices, float* values,
                                              int64_t* indptr_t, int32_t* indices_t, float* values_t,
                                              int32_t* deg, int32_t* halo_gid,
                                              int64_t* nnz_out, int64_t* n_halo_out,
                                              void* ws, size_t ws_bytes, void* stream) {
    if (!nnz_out || !n_halo_out) return fail(SAG_E_INVALID, "build: null size outputs");
    *nnz_out = 0;
    *n_halo_out = 0;
    SAG_TRY(check_build_inputs(src, dst, n_edges, n_global, lo, hi, flags));
    if (cap_nnz < 0 || cap_halo < 0) return fail(SAG_E_INVALID, "build: negative size");
    if (norm != SAG_NORM_GCN && norm != SAG_NORM_MEAN && norm != SAG_NORM_NONE)
        return fail(SAG_E_INVALID, "build: bad norm");
    if (!indptr) return fail(SAG_E_INVALID, "build: null indptr");
    if (cap_nnz > 0 && (!indices || !values)) return fail(SAG_E_INVALID, "build: null indices/values");
    const bool want_t = indptr_t || indices_t || values_t;
    if (want_t && (!indptr_t || (cap_nnz > 0 && (!indices_t || !values_t))))
        return fail(SAG_E_INVALID, "build: transpose outputs must be all given or all NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    Front f;
    SAG_TRY(build_front(src, dst, n_edges, n_global, lo, hi, flags, ws, ws_bytes, s, f));
    BuildWs& w = f.w;
    const BuildGeom& g = f.g;
    const int64_t n_local = g.n_local;
    const uint64_t nc = g.nc;
    uint64_t* uniq = f.uniq;
    const int64_t nnz = f.nnz, n_halo = f.n_halo;
    *nnz_out = nnz;
    *n_halo_out = n_halo;
    if (nnz > cap_nnz || n_halo > cap_halo)
        return fail(SAG_E_WORKSPACE, "build: output capacity too small (sizes returned)");
    if (n_halo > 0) {
        if (!halo_gid) return fail(SAG_E_INVALID, "build: halo nodes present but halo_gid is NULL");
        halo_list<<<grid_for(n_global), 256, 0, s>>>(w.flags, w.pos, n_global, halo_gid);
        SAG_LAUNCH_CHECK();
    }

    // 5. CSR arrays
    SAG_TRY(rows_from_sorted_keys(uniq, nnz, nc, n_local, indptr, s));
    if (nnz > 0) {
        final_columns<<<grid_for(nnz), 256, 0, s>>>(uniq, nnz, nc, n_local, w.pos, indices);
        SAG_LAUNCH_CHECK();
    }
    // 6. degrees (local rows, then halo columns)
    const int64_t n_ext = n_local + n_halo;
    if (n_local > 0) {
        row_degrees<<<grid_for(n_local), 256, 0, s>>>(indptr, n_local, w.deg);
        SAG_LAUNCH_CHECK();
    }
    if (n_halo > 0) {
        if (deg_global) {
            halo_degrees_given<<<grid_for(n_halo), 256, 0, s>>>(halo_gid, n_halo, deg_global, w.deg + n_local);
            SAG_LAUNCH_CHECK();
        } else {
            fill_i32<<<grid_for(n_halo), 256, 0, s>>>(w.deg + n_local, n_halo, 1);
            SAG_LAUNCH_CHECK();
            halo_degrees_count<<<grid_for(nnz), 256, 0, s>>>(indices, nnz, n_local, w.deg);
            SAG_LAUNCH_CHECK();
        }
    }
    if (deg && n_ext > 0)
        SAG_CHECK_HIP(hipMemcpyAsync(deg, w.deg, sizeof(int32_t) * n_ext, hipMemcpyDeviceToDevice, s));
    // 7. values
    if (nnz > 0) {
        values_a<<<grid_for(nnz), 256, 0, s>>>(uniq, nnz, nc, indices, w.deg, static_cast<int>(norm), values);
        SAG_LAUNCH_CHECK();
    }
    // 8. transpose: sort (column, row) keys
    if (want_t) {
        uint64_t* tk = uniq == w.keys_a ? w.keys_b : w.keys_a;
        uint64_t* other = uniq;   // the row-major keys are no longer needed after this kernel
        if (nnz > 0) {
            transpose_keys<<<grid_for(nnz), 256, 0, s>>>(uniq, nnz, nc, indices, n_local, tk);
            SAG_LAUNCH_CHECK();
        }
        const int tbits = bits_for(n_local > 0 && n_ext > 0
                                       ? static_cast<uint64_t>(n_ext) * static_cast<uint64_t>(n_local) - 1 : 0);
        uint64_t* tsorted = nullptr;
        SAG_TRY(radix_sort_u64(tk, other, nnz, tbits, w.tmp, w.tmp_bytes, s, &tsorted));
        SAG_TRY(rows_from_sorted_keys(tsorted, nnz, static_cast<uint64_t>(n_local > 0 ? n_local : 1),
                                      n_ext, indptr_t, s));
        if (nnz > 0) {
            transpose_fill<<<grid_for(nnz), 256, 0, s>>>(tsorted, nnz, n_local, w.deg, static_cast<int>(norm),
                                                         indices_t, values_t);
            SAG_LAUNCH_CHECK();
        }
    }
    SAG_CHECK_HIP(hipStreamSynchronize(s));
    return SAG_OK;
}
