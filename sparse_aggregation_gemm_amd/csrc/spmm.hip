// CSR SpMM Y = A X for the aggregation step of a GNN layer (CAGNET page:
// the A^T H product, one output row per CSR row; DIGEST: P_in H_in +
// P_out H~_out is one product over the columns [local | halo]).
//
// The product is bound by HBM bandwidth, so the kernels are built around
// 16-byte feature loads: a row of X is split into C = ceil(d / V) vectors of
// V elements (V = 4 fp32 or 8 bf16), and a group of G lanes (G = the power
// of two >= C, at most 64; wider rows give each lane NV vectors) covers one
// row of X.  A wavefront therefore holds P = 64 / G groups:
//   short rows  -- each group sums its own row (P rows per wavefront);
//   medium rows -- the wavefront sums one row, group g taking entries
//                  g, g + P, ...; the P partial sums are then added by a
//                  fixed butterfly;
//   long rows   -- one wavefront per segment of seg_len entries writes an
//                  fp32 partial row; a second kernel adds the partials of
//                  each row in segment order.
// Column indices and values are loaded cooperatively (one per lane) and
// handed to the group that needs them with lane shuffles, so each lane keeps
// several independent 16-byte loads in flight.  Accumulation is fp32 in a
// fixed order, so results are bitwise reproducible.
//
// A matrix with a hub split takes two passes: its hub part (the entries in
// the few columns holding the most entries) into fp32 partial rows, then its
// cold part, each row adding its partial before the epilogue.  During the
// first pass every gather lands on the same few rows of X, which stay in L2;
// on graphs with hundreds of entries per row that outweighs writing and
// reading the partial rows.
#include <mutex>

#include "ops.h"
#include "rowsum.h"
#include "trace.h"

namespace sag {
namespace {

using namespace rowsum;

constexpr int kWaves = 4;

template <class YT>
struct EpiArgs {
    YT* y;
    int64_t ldy;
    YT* pre;
    const YT* add;
    int64_t ld_add;
    int64_t n_add;
    const float* bias;
    int relu;
    int d;
    int row_mean;   // scale each row's sum by 1/len (values not read)
    const float* part;   // fp32 partial rows added to the sums first (or null)
    int64_t ld_part;
};

template <class XT, class YT>
struct SpArgs {
    const XT* X;
    int64_t ldx;
    int C;                    // 16-B vectors per row of X
    const int64_t* indptr;
    const int32_t* idx;
    const float* val;
    const int4* rec_short;    // row records of each bin
    const int4* rec_medium;   // (null: every row is medium, natural order)
    const int4* rec_long;
    int64_t n_short, n_medium, n_long, n_seg;
    int64_t nb_seg, nb_medium;  // workgroups of the segment and medium bins
    const int4* seg;          // segment records (long bin)
    const int32_t* seg0;      // segments per long row, prefix
    float* part;              // fp32 partial rows, ld = C * V
    int compact_long;         // long rows only: output row j of the long bin at row j
    EpiArgs<YT> e;
};

// The addend and bias of V consecutive outputs starting at column ch * V,
// loaded before the row's gathers so that their latency hides under them
// (read at the end of the row, they cost a full memory round trip per row).
// The addend is read as whole 16-byte vectors: the vector that holds the
// row's last element lies inside its pitch.  The bias has exactly d entries.
template <class YT, int V>
struct EpiIn {
    static constexpr int NU = V * static_cast<int>(sizeof(YT)) / 16;
    uint4 add[NU];
    float bias[V];
};

template <class YT, int V>
__device__ __forceinline__ void epi_load(const EpiArgs<YT>& e, int64_t row, int ch, bool live, EpiIn<YT, V>& in) {
    constexpr int VY = Vec<YT>::N;
    const int col0 = ch * V;
#pragma unroll
    for (int q = 0; q < EpiIn<YT, V>::NU; ++q) {
        in.add[q] = make_uint4(0, 0, 0, 0);
        if (live && e.add && row < e.n_add && col0 + q * VY < e.d)
            in.add[q] = *reinterpret_cast<const uint4*>(e.add + row * e.ld_add + col0 + q * VY);
    }
#pragma unroll
    for (int k = 0; k < V; ++k) in.bias[k] = live && e.bias && col0 + k < e.d ? e.bias[col0 + k] : 0.f;
}

// Epilogue and store of V consecutive outputs starting at column ch * V.
template <class YT, int V>
__device__ __forceinline__ void epi_store(const EpiArgs<YT>& e, int64_t row, int ch, float* a,
                                          const EpiIn<YT, V>& in, int len) {
    const int col0 = ch * V;
    if (col0 >= e.d) return;
    const int n = min(V, e.d - col0);
    constexpr int VY = Vec<YT>::N;
    if (e.part) {
        // the partial row of the hub pass, read here rather than with the
        // addend so that products without one hold no registers for it
        // (whole 16-byte vectors: ld_part is a multiple of 8; one at a time)
#pragma unroll 1
        for (int q = 0; q < V; q += 4) {
            if (col0 + q < e.d) {
                const float4 t = *reinterpret_cast<const float4*>(e.part + row * e.ld_part + col0 + q);
                a[q] += t.x;
                a[q + 1] += t.y;
                a[q + 2] += t.z;
                a[q + 3] += t.w;
            }
        }
    }
    if (e.row_mean && len > 0) {
        // the value the mean normalisation stores, 1/len rounded once
        const float rs = 1.f / static_cast<float>(len);
#pragma unroll
        for (int k = 0; k < V; ++k) a[k] *= rs;
    }
    if (e.add && row < e.n_add) {
        float t[V];
#pragma unroll
        for (int q = 0; q < EpiIn<YT, V>::NU; ++q) unpack<YT>(in.add[q], t + q * VY);
#pragma unroll
        for (int k = 0; k < V; ++k)
            if (k < n) a[k] += t[k];
    }
    if (e.bias) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            if (k < n) a[k] += in.bias[k];
    }
    if (e.pre) {
#pragma unroll
        for (int q = 0; q < V; q += VY) {
            const int nq = min(VY, n - q);
            if (nq > 0) store_vals<YT>(e.pre + row * e.ldy + col0 + q, a + q, nq);
        }
    }
    if (e.relu) {
#pragma unroll
        for (int k = 0; k < V; ++k) a[k] = a[k] < 0.f ? 0.f : a[k];
    }
#pragma unroll
    for (int q = 0; q < V; q += VY) {
        const int nq = min(VY, n - q);
        if (nq > 0) store_vals<YT>(e.y + row * e.ldy + col0 + q, a + q, nq);
    }
}

// ---- short rows: one group of G lanes per row -------------------------------
template <class XT, class YT, int G, int NV>
__device__ __forceinline__ void short_rows(const SpArgs<XT, YT>& p, int64_t block) {
    constexpr int V = Vec<XT>::N;
    constexpr int P = 64 / G;
    constexpr int U = NV >= 4 ? 2 : (NV >= 2 ? 4 : 8);
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    const int64_t i = (block * kWaves + (threadIdx.x >> 6)) * P + grp;
    const bool valid = i < p.n_short;
    int row = 0, len = 0;
    int64_t start = 0;
    if (valid) {
        const int4 r = p.rec_short[i];
        row = r.x;
        len = r.y;
        start = rec_start(r);
    }
    int lmax = len;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lmax = max(lmax, __shfl_xor(lmax, off, 64));
    int ch[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) ch[v] = min(v * G + gl, p.C - 1);
    // (rows of one vector per lane load the epilogue inputs first; wider
    // rows, with more work per row to hide the latency, at the end)
    EpiIn<YT, V> ein[NV];
    if constexpr (NV == 1) epi_load<YT, V>(p.e, row, gl, valid && gl < p.C, ein[0]);
    float acc[NV][V];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int k = 0; k < V; ++k) acc[v][k] = 0.f;

    for (int j0 = 0; j0 < lmax; j0 += G) {
        const int jj = j0 + gl;
        const bool mine = jj < len;
        const int32_t c_my = mine ? p.idx[start + jj] : 0;
        const float v_my = mine ? (p.val ? p.val[start + jj] : 1.f) : 0.f;
        const int nh = min(G, lmax - j0);
        for (int t = 0; t < nh; t += U) {
            int32_t c[U];
            float w[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int src = grp * G + min(t + u, G - 1);
                c[u] = __shfl(c_my, src, 64);
                w[u] = __shfl(v_my, src, 64);
                ok[u] = (t + u < nh) && (j0 + t + u < len);
            }
            accumulate<XT, NV, U>(p.X, p.ldx, ch, c, w, ok, acc);
        }
    }
    if (!valid) return;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int cv = v * G + gl;
        if constexpr (NV != 1) epi_load<YT, V>(p.e, row, cv, cv < p.C, ein[v]);
        if (cv < p.C) epi_store<YT, V>(p.e, row, cv, acc[v], ein[v], len);
    }
}

// ---- medium rows: one wavefront per row ----------------------------------------
template <class XT, class YT, int G, int NV>
__device__ __forceinline__ void medium_rows(const SpArgs<XT, YT>& p, int64_t block) {
    constexpr int V = Vec<XT>::N;
    const int64_t w = block * kWaves + (threadIdx.x >> 6);
    if (w >= p.n_medium) return;
    int64_t row, start;
    int len;
    if (p.rec_medium) {
        const int4 r = p.rec_medium[w];
        row = r.x;
        len = r.y;
        start = rec_start(r);
    } else {
        row = w;
        start = p.indptr[w];
        len = static_cast<int>(p.indptr[w + 1] - start);
    }
    const int lane = threadIdx.x & 63;
    EpiIn<YT, V> ein[NV];
    if constexpr (NV == 1) epi_load<YT, V>(p.e, row, lane, lane < G && lane < p.C, ein[0]);
    float acc[NV][V];
    wave_row_sum<XT, G, NV>(p.X, p.ldx, p.C, p.idx, p.val, start, len, acc);
    if (lane >= G) return;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int cv = v * G + lane;
        if constexpr (NV != 1) epi_load<YT, V>(p.e, row, cv, cv < p.C, ein[v]);
        if (cv < p.C) epi_store<YT, V>(p.e, row, cv, acc[v], ein[v], len);
    }
}

// ---- long rows: one wavefront per segment, fp32 partials -----------------------
template <class XT, class YT, int G, int NV>
__device__ __forceinline__ void segments(const SpArgs<XT, YT>& p, int64_t block) {
    constexpr int V = Vec<XT>::N;
    const int64_t sidx = block * kWaves + (threadIdx.x >> 6);
    if (sidx >= p.n_seg) return;
    const int4 sr = p.seg[sidx];
    const int64_t start = static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(sr.y)) |
                                               (static_cast<uint64_t>(static_cast<uint32_t>(sr.z)) << 32));
    float acc[NV][V];
    wave_row_sum<XT, G, NV>(p.X, p.ldx, p.C, p.idx, p.val, start, sr.w, acc);
    const int lane = threadIdx.x & 63;
    if (lane >= G) return;
    float* out = p.part + sidx * static_cast<int64_t>(p.C) * V;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int cv = v * G + lane;
        if (cv < p.C) {
#pragma unroll
            for (int q = 0; q < V; q += 4)
                *reinterpret_cast<float4*>(out + cv * V + q) =
                    make_float4(acc[v][q], acc[v][q + 1], acc[v][q + 2], acc[v][q + 3]);
        }
    }
}

// All three bins in one launch: the workgroups of long-row segments come
// first (the longest work starts first), then medium rows, then short rows.
template <class XT, class YT, int G, int NV>
__device__ __forceinline__ void bins(const SpArgs<XT, YT>& p) {
    int64_t b = blockIdx.x;
    if (b < p.nb_seg) {
        segments<XT, YT, G, NV>(p, b);
        return;
    }
    b -= p.nb_seg;
    if (b < p.nb_medium) {
        medium_rows<XT, YT, G, NV>(p, b);
        return;
    }
    short_rows<XT, YT, G, NV>(p, b - p.nb_medium);
}

template <class XT, class YT, int G, int NV>
__global__ __launch_bounds__(256) void spmm_bins(SpArgs<XT, YT> p) {
    bins<XT, YT, G, NV>(p);
}

// One 128-byte column slice of every row (eight lanes of one 16-byte vector
// each): the same code as spmm_bins<XT, YT, 8, 1>, under a name of its own so
// that a profile tells slice passes from whole narrow rows.
template <class XT, class YT>
__global__ __launch_bounds__(256) void spmm_slice(SpArgs<XT, YT> p) {
    bins<XT, YT, 8, 1>(p);
}

// Adds the partial rows of each long row in segment order, then the epilogue.
template <class XT, class YT>
__global__ __launch_bounds__(256) void spmm_long_reduce(SpArgs<XT, YT> p) {
    constexpr int V = Vec<XT>::N;
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (j >= p.n_long) return;
    const int lane = threadIdx.x & 63;
    const int64_t row = p.compact_long ? j : p.rec_long[j].x;
    const int len = p.rec_long[j].y;
    const int32_t s0 = p.seg0[j], s1 = p.seg0[j + 1];
    const int64_t ldp = static_cast<int64_t>(p.C) * V;
    for (int ch = lane; ch < p.C; ch += 64) {
        EpiIn<YT, V> ein;
        epi_load<YT, V>(p.e, row, ch, true, ein);
        float a[V];
#pragma unroll
        for (int k = 0; k < V; ++k) a[k] = 0.f;
        for (int32_t s = s0; s < s1; ++s) {
            const float* src = p.part + s * ldp + ch * V;
#pragma unroll
            for (int q = 0; q < V; q += 4) {
                const float4 t = *reinterpret_cast<const float4*>(src + q);
                a[q] += t.x;
                a[q + 1] += t.y;
                a[q + 2] += t.z;
                a[q + 3] += t.w;
            }
        }
        epi_store<YT, V>(p.e, row, ch, a, ein, len);
    }
}

template <class XT, class YT, int G, int NV>
sag_status launch_bins(const sag_csr& A, SpArgs<XT, YT> p, hipStream_t s, bool long_only, bool slice = false) {
    constexpr int P = 64 / G;
    const int4* rec = reinterpret_cast<const int4*>(A.sched);
    if (!rec) {
        p.rec_medium = nullptr;
        p.n_medium = A.n_rows;
    } else {
        p.rec_short = rec;
        p.n_short = A.n_short;
        p.rec_medium = rec + A.n_short;
        p.n_medium = A.n_medium;
        p.rec_long = rec + A.n_short + A.n_medium;
        p.n_long = A.n_long;
        p.seg = rec + A.n_rows;
        p.seg0 = reinterpret_cast<const int32_t*>(rec + A.n_rows + A.n_seg);
        p.n_seg = A.n_long > 0 ? A.n_seg : 0;
    }
    if (long_only) {
        if (!rec) return SAG_OK;
        p.n_short = p.n_medium = 0;
        p.compact_long = 1;
    }
    p.nb_seg = cdiv(p.n_seg, kWaves);
    p.nb_medium = cdiv(p.n_medium, kWaves);
    const int64_t nb_short = cdiv(p.n_short, kWaves * P);
    const int64_t blocks = p.nb_seg + p.nb_medium + nb_short;
    if (blocks > 0) {
        if constexpr (G == 8 && NV == 1) {
            if (slice)
                spmm_slice<XT, YT><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(p);
            else
                spmm_bins<XT, YT, G, NV><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(p);
        } else {
            spmm_bins<XT, YT, G, NV><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(p);
        }
        SAG_LAUNCH_CHECK();
    }
    if (p.n_long > 0) {
        spmm_long_reduce<XT, YT><<<dim3(static_cast<unsigned>(cdiv(p.n_long, kWaves))), 256, 0, s>>>(p);
        SAG_LAUNCH_CHECK();
    }
    return SAG_OK;
}

template <class XT, class YT>
sag_status run_typed(const sag_csr& A, const void* X, int64_t ldx, int64_t d, void* Y, int64_t ldy,
                     const Epilogue& epi, void* ws, hipStream_t s, bool long_only = false, bool slice = false) {
    constexpr int V = Vec<XT>::N;
    SpArgs<XT, YT> p{};
    p.X = static_cast<const XT*>(X);
    p.ldx = ldx;
    p.C = static_cast<int>(cdiv(d, V));
    p.indptr = A.indptr;
    p.idx = A.indices;
    p.val = epi.row_mean ? nullptr : A.values;
    p.part = static_cast<float*>(ws);
    p.e.y = static_cast<YT*>(Y);
    p.e.ldy = ldy;
    p.e.pre = static_cast<YT*>(epi.pre);
    p.e.add = static_cast<const YT*>(epi.addend);
    p.e.ld_add = epi.ld_add;
    p.e.n_add = epi.n_add;
    p.e.bias = epi.bias;
    p.e.relu = epi.relu;
    p.e.d = static_cast<int>(d);
    p.e.row_mean = epi.row_mean;
    p.e.part = epi.part;
    p.e.ld_part = epi.ld_part;
    const int C = p.C;
    if (slice) {
        if (C > 8) return fail(SAG_E_INVALID, "spmm: a column slice spans more than 128 bytes");
        return launch_bins<XT, YT, 8, 1>(A, p, s, long_only, true);
    }
    if (C <= 4) return launch_bins<XT, YT, 4, 1>(A, p, s, long_only);
    if (C <= 8) return launch_bins<XT, YT, 8, 1>(A, p, s, long_only);
    if (C <= 16) return launch_bins<XT, YT, 16, 1>(A, p, s, long_only);
    if (C <= 32) return launch_bins<XT, YT, 32, 1>(A, p, s, long_only);
    if (C <= 64) return launch_bins<XT, YT, 64, 1>(A, p, s, long_only);
    if (C <= 128) return launch_bins<XT, YT, 64, 2>(A, p, s, long_only);
    if (C <= 192) return launch_bins<XT, YT, 64, 3>(A, p, s, long_only);
    if (C <= 256) return launch_bins<XT, YT, 64, 4>(A, p, s, long_only);
    return fail(SAG_E_UNSUPPORTED, "spmm: row width above 256 vectors of 16 bytes");
}

}  // namespace

sag_status spmm_long_run(const sag_csr& A, const void* X, int64_t ldx, sag_dtype dt, int64_t d, void* Y, int64_t ldy,
                         void* ws, size_t ws_bytes, hipStream_t s) {
    if (!A.sched || A.n_long == 0 || d == 0) return SAG_OK;
    if (ws_bytes < spmm_long_ws_bytes(A, d) || !ws) return fail(SAG_E_WORKSPACE, "spmm: workspace too small");
    Epilogue e;
    e.row_mean = A.row_mean != 0;
    if (dt == SAG_BF16) return run_typed<uint16_t, uint16_t>(A, X, ldx, d, Y, ldy, e, ws, s, true);
    return run_typed<float, float>(A, X, ldx, d, Y, ldy, e, ws, s, true);
}

sag_status check_csr(const char* name, const sag_csr* A) {
    const std::string n(name);
    if (!A) return fail(SAG_E_INVALID, n + ": null CSR");
    if (A->n_rows < 0 || A->n_cols < 0 || A->nnz < 0) return fail(SAG_E_INVALID, n + ": negative CSR size");
    if (A->n_rows > INT32_MAX || A->n_cols > INT32_MAX) return fail(SAG_E_INVALID, n + ": CSR too large for int32 ids");
    if (A->n_rows > 0 && !A->indptr) return fail(SAG_E_INVALID, n + ": null indptr");
    if (A->nnz > 0 && !A->indices) return fail(SAG_E_INVALID, n + ": null indices");
    if (A->nnz > 0 && A->n_cols == 0) return fail(SAG_E_INVALID, n + ": entries but no columns");
    if (A->sched) {
        if (A->n_short < 0 || A->n_medium < 0 || A->n_long < 0 || A->n_seg < 0 ||
            A->n_short + A->n_medium + A->n_long != A->n_rows)
            return fail(SAG_E_INVALID, n + ": inconsistent schedule counts");
        if (A->n_long > 0 && (A->n_seg < A->n_long || A->seg_len < 64))
            return fail(SAG_E_INVALID, n + ": inconsistent long-row schedule");
        if (!aligned16(A->sched)) return fail(SAG_E_ALIGN, n + ": schedule not 16-B aligned");
    }
    if (A->hub_part || A->cold_part) {
        if (!A->hub_part || !A->cold_part) return fail(SAG_E_INVALID, n + ": a hub split needs both parts");
        if (A->hub_part->hub_part || A->hub_part->cold_part)
            return fail(SAG_E_INVALID, n + ": the hub part of a hub split has a split (only the cold part may)");
        for (const sag_csr* P : {A->hub_part, A->cold_part}) {
            SAG_TRY(check_csr(name, P));
            if (P->n_rows != A->n_rows || P->n_cols != A->n_cols)
                return fail(SAG_E_INVALID, n + ": the parts of a hub split must have the matrix's shape");
            if (P->row_mean) return fail(SAG_E_INVALID, n + ": the parts of a hub split carry their values (row_mean 0)");
            if (A->values && P->nnz > 0 && !P->values)
                return fail(SAG_E_INVALID, n + ": the parts of a matrix with values must carry them");
        }
        if (A->hub_part->nnz + A->cold_part->nnz != A->nnz)
            return fail(SAG_E_INVALID, n + ": the parts of a hub split must hold the matrix's entries");
        if (A->row_mean && !A->values)
            return fail(SAG_E_INVALID, n + ": a row_mean matrix with a hub split must store its values");
    }
    return SAG_OK;
}

size_t spmm_long_ws_bytes(const sag_csr& A, int64_t d) {
    if (!A.sched || A.n_long == 0) return 0;
    const int64_t C = cdiv(d, 4);   // fp32 partials: C4 = ceil(d / 4) float4 vectors at most
    return static_cast<size_t>(A.n_seg) * static_cast<size_t>(round_up(C * 4, 8)) * sizeof(float);
}

// fp32 partial rows of a split product: round_up(d, 8) floats per row, so
// that the epilogue reads them as whole 16-byte vectors
static int64_t part_ld(int64_t d) { return round_up(d > 0 ? d : 1, 8); }
static size_t part_bytes(const sag_csr& A, int64_t d) {
    return static_cast<size_t>(round_up(A.n_rows * part_ld(d) * static_cast<int64_t>(sizeof(float)), 256));
}

// Hub groups of a split matrix (the length of its chain; 0 without a split).
static int chain_levels(const sag_csr& A) {
    int k = 0;
    for (const sag_csr* M = &A; M->hub_part && M->cold_part; M = M->cold_part) ++k;
    return k;
}

// A split matrix: partial rows (two buffers used in turn along a chain of
// several groups), then the largest long-row need of any pass.
size_t spmm_ws_bytes(const sag_csr& A, int64_t d) {
    const int levels = chain_levels(A);
    if (levels == 0) return spmm_long_ws_bytes(A, d);
    size_t lw = 0;
    const sag_csr* M = &A;
    for (; M->hub_part && M->cold_part; M = M->cold_part) {
        const size_t h = spmm_long_ws_bytes(*M->hub_part, d);
        lw = h > lw ? h : lw;
    }
    const size_t c = spmm_long_ws_bytes(*M, d);
    lw = c > lw ? c : lw;
    return (levels > 1 ? 2 : 1) * part_bytes(A, d) + lw;
}

namespace {

sag_status spmm_dispatch(const sag_csr& A, const void* X, int64_t ldx, sag_dtype xt, int64_t d, void* Y,
                         int64_t ldy, sag_dtype yt, const Epilogue& epi, void* ws, hipStream_t s,
                         bool slice = false) {
    if (xt == SAG_F32 && yt == SAG_F32) return run_typed<float, float>(A, X, ldx, d, Y, ldy, epi, ws, s, false, slice);
    if (xt == SAG_BF16 && yt == SAG_BF16)
        return run_typed<uint16_t, uint16_t>(A, X, ldx, d, Y, ldy, epi, ws, s, false, slice);
    if (xt == SAG_BF16 && yt == SAG_F32)
        return run_typed<uint16_t, float>(A, X, ldx, d, Y, ldy, epi, ws, s, false, slice);
    return fail(SAG_E_UNSUPPORTED, "spmm: unsupported (X, Y) dtype pair");
}

constexpr int64_t kSliceBytes = 128;   // one cache line of each row per pass

// The one-pass product, or, when A asks for column slices and a row of X
// spans more than two of them, one pass per 128-byte column slice of X (the
// last narrower) writing the same columns of Y: each pass gathers one line
// per entry, so L2 holds the lines of four times as many rows of X.  The
// epilogue is per element, so each slice takes its own columns of the
// addend, bias and Y_pre.  Every slice reuses the long-row partials (stream
// order: a slice's reduce finishes before the next slice's segments write).
sag_status spmm_one_pass(const sag_csr& A, const void* X, int64_t ldx, sag_dtype xt, int64_t d, void* Y,
                         int64_t ldy, sag_dtype yt, const Epilogue& epi, void* ws, hipStream_t s) {
    const int64_t ex = elt_size(xt), ey = elt_size(yt);
    if (!A.col_slices || d * ex <= 2 * kSliceBytes) return spmm_dispatch(A, X, ldx, xt, d, Y, ldy, yt, epi, ws, s);
    const int64_t w = kSliceBytes / ex;
    for (int64_t c0 = 0; c0 < d; c0 += w) {
        Epilogue e = epi;
        if (e.addend) e.addend = static_cast<const char*>(e.addend) + c0 * ey;
        if (e.bias) e.bias += c0;
        if (e.pre) e.pre = static_cast<char*>(e.pre) + c0 * ey;
        SAG_TRY(spmm_dispatch(A, static_cast<const char*>(X) + c0 * ex, ldx, xt, w < d - c0 ? w : d - c0,
                              static_cast<char*>(Y) + c0 * ey, ldy, yt, e, ws, s, true));
    }
    return SAG_OK;
}

}  // namespace

// The product over A with epi.  A split matrix: one pass per hub group into
// fp32 partial rows (the parts carry their values), each adding the previous
// group's partial rows (two buffers used in turn), then the pass over the
// final cold part with the last partial rows added before the epilogue.
static sag_status spmm_chain(const sag_csr& A, const void* X, int64_t ldx, sag_dtype xt, int64_t d, void* Y,
                             int64_t ldy, sag_dtype yt, const Epilogue& epi, void* ws, hipStream_t s) {
    const int levels = chain_levels(A);
    if (levels == 0) return spmm_one_pass(A, X, ldx, xt, d, Y, ldy, yt, epi, ws, s);
    const size_t pb = part_bytes(A, d);
    char* base = static_cast<char*>(ws);
    void* lws = base + (levels > 1 ? 2 : 1) * pb;
    const int64_t ldp = part_ld(d);
    const float* prev = nullptr;
    const sag_csr* M = &A;
    for (int k = 0; M->hub_part && M->cold_part; M = M->cold_part, ++k) {
        float* P = reinterpret_cast<float*>(base + (k % 2) * pb);
        Epilogue e1;
        e1.part = prev;
        e1.ld_part = ldp;
        SAG_TRY(spmm_dispatch(*M->hub_part, X, ldx, xt, d, P, ldp, SAG_F32, e1, lws, s));
        prev = P;
    }
    Epilogue e2 = epi;
    e2.row_mean = 0;
    e2.part = prev;
    e2.ld_part = ldp;
    return spmm_dispatch(*M, X, ldx, xt, d, Y, ldy, yt, e2, lws, s);
}

sag_status spmm_run(const sag_csr& A, const void* X, int64_t ldx, sag_dtype xt, int64_t d, void* Y,
                    int64_t ldy, sag_dtype yt, const Epilogue& epi, void* ws, size_t ws_bytes,
                    hipStream_t s) {
    if (A.n_rows == 0 || d == 0) return SAG_OK;
    if (ws_bytes < spmm_ws_bytes(A, d) || (spmm_ws_bytes(A, d) > 0 && !ws))
        return fail(SAG_E_WORKSPACE, "spmm: workspace too small");
    // algorithmic bytes of the product itself: CSR arrays once (values only
    // when read), every X row once, every output row once; the epilogue's
    // addend and Y_pre are not counted
    const int64_t ex = elt_size(xt), ey = elt_size(yt);
    const int64_t bytes = 8 * (A.n_rows + 1) + A.nnz * (A.values && !epi.row_mean ? 8 : 4) + ex * d * A.n_cols +
                          ey * d * A.n_rows;
    TraceScope trace(trace_enabled() ? shape_name("spmm", xt == SAG_BF16 ? (yt == SAG_BF16 ? "bf16" : "bf16>f32") : "f32",
                                                  A.n_rows, A.nnz, d)
                                     : std::string(),
                     s, bytes, 2 * A.nnz * d);
    return spmm_chain(A, X, ldx, xt, d, Y, ldy, yt, epi, ws, s);
}

}  // namespace sag

using namespace sag;

extern "C" size_t sag_spmm_workspace_bytes(const sag_csr* A, int64_t d) {
    if (!A || d < 0) return 0;
    return spmm_ws_bytes(*A, d);
}

static sag_status spmm_check(const char* name, const sag_csr* A, const void* X, int64_t ldx, sag_dtype xt,
                             int64_t d, void* Y, int64_t ldy, sag_dtype yt, const void* addend,
                             int64_t ld_add, int64_t n_add) {
    SAG_TRY(check_csr(name, A));
    if (d < 0) return fail(SAG_E_INVALID, std::string(name) + ": negative width");
    const int64_t maxd = xt == SAG_BF16 ? 2048 : 1024;
    if (d > maxd) return fail(SAG_E_UNSUPPORTED, std::string(name) + ": width too large");
    SAG_TRY(check_dense("spmm X", X, A->nnz > 0 ? A->n_cols : 0, d, ldx, xt));
    SAG_TRY(check_dense("spmm Y", Y, A->n_rows, d, ldy, yt));
    if (n_add < 0 || n_add > A->n_rows) return fail(SAG_E_INVALID, std::string(name) + ": n_add out of range");
    if (addend) SAG_TRY(check_dense("spmm addend", addend, n_add, d, ld_add, yt));
    if (!(xt == SAG_F32 && yt == SAG_F32) && !(xt == SAG_BF16 && yt == SAG_BF16) &&
        !(xt == SAG_BF16 && yt == SAG_F32))
        return fail(SAG_E_UNSUPPORTED, std::string(name) + ": unsupported (X, Y) dtype pair");
    return SAG_OK;
}

static Epilogue entry_epilogue(const sag_csr* A, const void* addend, int64_t ld_add, int64_t n_add) {
    Epilogue e;
    e.addend = addend;
    e.ld_add = ld_add;
    e.n_add = addend ? n_add : 0;
    e.row_mean = A->row_mean != 0;
    return e;
}

static sag_status spmm_entry(const char* name, const sag_csr* A, const void* X, int64_t ldx, sag_dtype xt,
                             int64_t d, void* Y, int64_t ldy, sag_dtype yt, const void* addend,
                             int64_t ld_add, int64_t n_add, void* ws, size_t ws_bytes, void* stream) {
    SAG_TRY(spmm_check(name, A, X, ldx, xt, d, Y, ldy, yt, addend, ld_add, n_add));
    return spmm_run(*A, X, ldx, xt, d, Y, ldy, yt, entry_epilogue(A, addend, ld_add, n_add), ws, ws_bytes,
                    static_cast<hipStream_t>(stream));
}

extern "C" sag_status sag_spmm_csr(const sag_csr* A, const void* X, int64_t ldx, sag_dtype xt, int64_t d,
                                   void* Y, int64_t ldy, sag_dtype yt, const void* addend, int64_t ld_add,
                                   int64_t n_add, void* ws, size_t ws_bytes, void* stream) {
    return spmm_entry("spmm_csr", A, X, ldx, xt, d, Y, ldy, yt, addend, ld_add, n_add, ws, ws_bytes, stream);
}

extern "C" sag_status sag_spmm_csr_t(const sag_csr* AT, const void* X, int64_t ldx, sag_dtype xt, int64_t d,
                                     void* Y, int64_t ldy, sag_dtype yt, const void* addend, int64_t ld_add,
                                     int64_t n_add, void* ws, size_t ws_bytes, void* stream) {
    return spmm_entry("spmm_csr_t", AT, X, ldx, xt, d, Y, ldy, yt, addend, ld_add, n_add, ws, ws_bytes, stream);
}

// ---- allocation-free variant ------------------------------------------------------
// The long-row partials of sag_spmm_csr_noalloc live in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not the device address: the address comes from
// hipGetSymbolAddress, once per device, and only that pointer is handed to
// kernels.
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on its first use on
// that device).
sag_status scratch_address(void** out) {
    int dev = -1;
    SAG_CHECK_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(SAG_E_UNSUPPORTED, "spmm_csr_noalloc: device ordinal too large");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        SAG_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(SAG_E_HIP, "spmm_csr_noalloc: no device address for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SAG_OK;
}

}  // namespace

extern "C" size_t sag_spmm_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" sag_status sag_spmm_csr_noalloc(const sag_csr* A, const void* X, int64_t ldx, sag_dtype xt, int64_t d,
                                           void* Y, int64_t ldy, sag_dtype yt, const void* addend,
                                           int64_t ld_add, int64_t n_add, void* stream) {
    SAG_TRY(spmm_check("spmm_csr_noalloc", A, X, ldx, xt, d, Y, ldy, yt, addend, ld_add, n_add));
    const size_t need = spmm_long_ws_bytes(*A, d);   // one pass: a hub split is not used here
    if (need > kScratchBytes)
        return fail(SAG_E_WORKSPACE, "spmm_csr_noalloc: the long rows' partial sums need " + std::to_string(need) +
                                         " bytes, above the fixed scratch of " + std::to_string(kScratchBytes) +
                                         " bytes (use sag_spmm_csr with a workspace)");
    if (A->n_rows == 0 || d == 0) return SAG_OK;
    void* ws = nullptr;
    if (need > 0) SAG_TRY(scratch_address(&ws));
    return spmm_one_pass(*A, X, ldx, xt, d, Y, ldy, yt, entry_epilogue(A, addend, ld_add, n_add), ws,
                         static_cast<hipStream_t>(stream));
}
