// Fused aggregate -> transform: one kernel sums rows of A H_ext into an LDS
// tile and multiplies the tile by W on the matrix cores, so the aggregate
// does not make a round trip through HBM between an SpMM and a GEMM (the
// CAGNET page's local SpMM followed by the dense product with W; the
// product here consumes the SpMM's tile where it was formed).
//
//   GCN        : Out = act(Z W + b),              Z = A H_ext
//   GraphSAGE  : Out = act([H_local | Z] W + b)   (own row first)
// Z is also stored when the caller keeps it (the backward pass reads it).
//
// A workgroup of eight wavefronts takes 32 consecutive row records of A's
// schedule, last records first (so the longest rows start first).  Each
// wavefront sums 4 of the rows: short rows (<= 32 entries) with a group of
// lanes per row, several rows at a time (rowsum::group_row_sum), longer
// rows one after another with the whole wavefront (rowsum::wave_row_sum).
// Each sum is rounded to the storage type (the value a separate SpMM would
// store) and written into the tile, and into Z.  The
// wavefronts then split the output columns in blocks of 32 and run
// v_mfma_f32_32x32x16_bf16 (fp32: v_mfma_f32_32x32x2f32) over K, with the
// tile as the B operand (C^T = W^T tile^T, so a lane ends with one output
// row) and W read from a fragment-ordered copy that stays in L2: one 16-byte
// load per lane per k-group, K x N elements per 32 rows.  The results go
// through LDS and leave as whole 16-byte row vectors.  Rows the schedule
// cuts into segments are summed beforehand by the SpMM's segment kernels
// into a compact buffer, from which the tile loads them.
#include <algorithm>

#include "ops.h"
#include "rowsum.h"
#include "trace.h"

namespace sag {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;          // rows per tile (one MFMA block)
// Eight wavefronts per tile: each sums four rows and owns one output block
// (four wavefronts, eight rows each, ran 6% slower at 3 waves per SIMD).
constexpr int kTileWaves = 8;
constexpr int kThreads = 64 * kTileWaves;
constexpr int kMaxNB = 8;          // output column blocks of 32 (N <= 256)

// Elements of one MFMA k-group held as 16 bytes per lane (two lane halves).
template <class T> constexpr int kgroup() { return sizeof(T) == 2 ? 16 : 8; }

template <class T>
struct FusedArgs {
    const int64_t* indptr;
    const int32_t* idx;
    const float* val;          // null: unit values (a row-mean CSR's pattern)
    int row_mean;              // scale each summed row by 1/len (values not read)
    const int4* rec;           // schedule records (null: natural row order)
    int64_t n_rows;
    int64_t n_summed;          // records [0, n_summed) are summed here, the rest are long rows
    const T* X;                // H_ext
    int64_t ldx;
    int C;                     // 16-byte vectors of a row of X
    int d;                     // d_in
    const T* self;             // GraphSAGE: own rows (null: GCN)
    int64_t ldself;
    const T* zlong;            // compact sums of the long rows
    int64_t ldzl;
    T* Z;                      // nullable
    int64_t ldz;
    const uint4* Bp;           // fragment-ordered W
    int kgroups;               // K / kgroup
    int NB;                    // output column blocks
    int koff;                  // first tile column of Z (0 GCN, round_up(d, V) GraphSAGE)
    int kvalid;                // koff + C * V: tile columns written per row
    int pitch;                 // tile row pitch (elements)
    int opitch;                // output staging row pitch (elements)
    int N;
    const float* bias;
    int relu;
    T* Y;
    T* pre;
    int64_t ldy;
    int64_t n_tiles;
    int64_t n_short;           // records [0, n_short) are short rows (schedule)
};

__device__ __forceinline__ int64_t rec_start(const int4& r) {
    return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(r.z)) |
                                (static_cast<uint64_t>(static_cast<uint32_t>(r.w)) << 32));
}

// Zeroes the elements of a 16-byte vector at or beyond `keep` (0..V).
template <class T>
__device__ __forceinline__ void zero_tail(float* f, int keep) {
#pragma unroll
    for (int k = 0; k < Vec<T>::N; ++k)
        if (k >= keep) f[k] = 0.f;
}

template <class T>
__device__ __forceinline__ uint4 pack_vec(const float* f) {
    if constexpr (sizeof(T) == 2) {
        uint4 o;
        o.x = uint32_t(f32_to_bf16(f[0])) | (uint32_t(f32_to_bf16(f[1])) << 16);
        o.y = uint32_t(f32_to_bf16(f[2])) | (uint32_t(f32_to_bf16(f[3])) << 16);
        o.z = uint32_t(f32_to_bf16(f[4])) | (uint32_t(f32_to_bf16(f[5])) << 16);
        o.w = uint32_t(f32_to_bf16(f[6])) | (uint32_t(f32_to_bf16(f[7])) << 16);
        return o;
    } else {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                          __float_as_uint(f[3]));
    }
}

template <class T, int G, int NV>
__global__ __launch_bounds__(kThreads) void agg_transform(FusedArgs<T> p) {
    constexpr int V = Vec<T>::N;
    constexpr int KG = kgroup<T>();
    extern __shared__ uint4 lds[];
    __shared__ int64_t rows_of[kRows];
    T* tile = reinterpret_cast<T*>(lds);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int gl = lane % G;
    const int64_t t = p.n_tiles - 1 - blockIdx.x;

    // ---- sums of the tile's rows (and own rows) into LDS.  A tile that
    // starts among the short rows gives each row a group of G lanes (P rows
    // per wavefront at a time); other tiles give each row the whole wavefront.
    // (a wavefront owns 8 rows; with more than 8 groups the extra groups idle)
    constexpr int kOwn = kRows / kTileWaves;
    constexpr int P = 64 / G;
    constexpr int kPer = P < kOwn ? P : kOwn;
    static_assert(kOwn % kPer == 0, "rows per wavefront must split into whole rounds");
    const bool group_mode = p.rec && t * kRows < p.n_short;
    const int rounds = group_mode ? kOwn / kPer : kOwn;
    const int grp = lane / G;
    const bool active = !group_mode || grp < kPer;
    if (threadIdx.x < kRows) rows_of[threadIdx.x] = -1;
    __syncthreads();
    for (int q = 0; q < rounds; ++q) {
        const int r = wave * kOwn + (group_mode ? q * kPer + (active ? grp : 0) : q);
        const int64_t i = active ? t * kRows + r : INT64_MAX;
        T* trow = tile + r * p.pitch;
        int64_t row = -1, start = 0;
        int len = 0;
        if (i < p.n_rows) {
            if (p.rec) {
                const int4 rc = p.rec[i];
                row = rc.x;
                len = rc.y;
                start = rec_start(rc);
            } else {
                row = i;
                start = p.indptr[i];
                len = static_cast<int>(p.indptr[i + 1] - start);
            }
        }
        const bool summed = i < p.n_summed;
        float acc[NV][V];
        if (group_mode) {
            const int mylen = summed ? len : 0;
            int lmax = mylen;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) lmax = max(lmax, __shfl_xor(lmax, off, 64));
            rowsum::group_row_sum<T, G, NV>(p.X, p.ldx, p.C, p.idx, p.val, start, mylen, lmax, acc);
        } else if (summed) {
            rowsum::wave_row_sum<T, G, NV>(p.X, p.ldx, p.C, p.idx, p.val, start, len, acc);
        }
        if (summed && p.row_mean && len > 0) {
            // the value the mean normalisation stores, 1/len rounded once
            const float rs = 1.f / static_cast<float>(len);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int k = 0; k < V; ++k) acc[v][k] *= rs;
        }
        if (row >= 0 && !summed) {
            const int64_t j = i - p.n_summed;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int ch = min(v * G + gl, p.C - 1);
                unpack<T>(*reinterpret_cast<const uint4*>(p.zlong + j * p.ldzl + ch * V), acc[v]);
            }
        }
        const bool writer = group_mode || lane < G;
        if (!active) {
            // idle group: touches nothing
        } else if (row >= 0) {
            if (writer) {
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int cv = v * G + gl;
                    if (cv >= p.C) continue;
                    const int col0 = cv * V;
                    zero_tail<T>(acc[v], p.d - col0);
                    const uint4 o = pack_vec<T>(acc[v]);
                    *reinterpret_cast<uint4*>(trow + p.koff + col0) = o;
                    if (p.Z) {
                        T* zp = p.Z + row * p.ldz + col0;
                        if (col0 + V <= p.d) {
                            *reinterpret_cast<uint4*>(zp) = o;
                        } else {
                            float f[V];
                            unpack<T>(o, f);
                            store_vals<T>(zp, f, p.d - col0);
                        }
                    }
                }
            }
            if (p.self) {
                const int gl2 = group_mode ? gl : lane;
                const int step = group_mode ? G : 64;
                for (int cv = gl2; cv < p.C; cv += step) {
                    float f[V];
                    unpack<T>(*reinterpret_cast<const uint4*>(p.self + row * p.ldself + cv * V), f);
                    zero_tail<T>(f, p.d - cv * V);
                    *reinterpret_cast<uint4*>(trow + cv * V) = pack_vec<T>(f);
                }
            }
            // the columns past the last vector up to the next k-group
            if ((group_mode ? gl : lane) == 0 && p.kvalid % KG != 0)
                *reinterpret_cast<uint4*>(trow + p.kvalid) = make_uint4(0, 0, 0, 0);
        } else {
            const int gl2 = group_mode ? gl : lane;
            const int step = group_mode ? G : 64;
            for (int c = gl2 * V; c < p.kgroups * KG; c += step * V)
                *reinterpret_cast<uint4*>(trow + c) = make_uint4(0, 0, 0, 0);
        }
        if (active && (group_mode ? gl : lane) == 0) rows_of[r] = row;
    }
    __syncthreads();

    // ---- tile x W: wave w takes column blocks w, w + waves, ...; then bias and
    // one rounding, staged through LDS (the tile's own space, once every
    // wavefront has read it): lane holds row lane % 32, columns
    // nb * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4
    const T* arow = tile + (lane & 31) * p.pitch + (KG / 2) * (lane >> 5);
    constexpr int kBlocks = (kMaxNB + kTileWaves - 1) / kTileWaves;   // column blocks per wavefront
    f32x16_t acc[kBlocks];
    bool has[kBlocks];
    const uint4* bk[kBlocks];
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
        has[j] = wave + j * kTileWaves < p.NB;
        bk[j] = p.Bp + static_cast<int64_t>(wave + j * kTileWaves) * 64 + lane;
    }
    const int64_t kstride = static_cast<int64_t>(p.NB) * 64;
    // W fragments of kPre k-groups are loaded together (their L2 latency is
    // paid once per kPre MFMA steps; deeper prefetch only costs registers)
    constexpr int kPre = 2;
    for (int kg0 = 0; kg0 < p.kgroups; kg0 += kPre) {
        uint4 b[kBlocks][kPre];
#pragma unroll
        for (int j = 0; j < kBlocks; ++j)
#pragma unroll
            for (int u = 0; u < kPre; ++u)
                b[j][u] = (has[j] && kg0 + u < p.kgroups) ? bk[j][(kg0 + u) * kstride] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            if (kg0 + u >= p.kgroups) break;
            const uint4 a = *reinterpret_cast<const uint4*>(arow + (kg0 + u) * KG);
#pragma unroll
            for (int j = 0; j < kBlocks; ++j) {
                if (!has[j]) continue;
                if constexpr (sizeof(T) == 2) {
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b[j][u]),
                                                                     __builtin_bit_cast(bf16x8_t, a), acc[j], 0, 0, 0);
                } else {
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j][u].x), __uint_as_float(a.x),
                                                                  acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j][u].y), __uint_as_float(a.y),
                                                                  acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j][u].z), __uint_as_float(a.z),
                                                                  acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(b[j][u].w), __uint_as_float(a.w),
                                                                  acc[j], 0, 0, 0);
                }
            }
        }
    }
    __syncthreads();
    T* otile = tile;
    const int m = lane & 31;
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
        const int nb = wave + j * kTileWaves;
        if (nb >= p.NB) continue;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int n0 = nb * 32 + 8 * g + 4 * (lane >> 5);
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + e;
                y[e] = acc[j][4 * g + e] + ((p.bias && n < p.N) ? p.bias[n] : 0.f);
            }
            if constexpr (sizeof(T) == 2) {
                uint2 o;
                o.x = uint32_t(f32_to_bf16(y[0])) | (uint32_t(f32_to_bf16(y[1])) << 16);
                o.y = uint32_t(f32_to_bf16(y[2])) | (uint32_t(f32_to_bf16(y[3])) << 16);
                *reinterpret_cast<uint2*>(otile + m * p.opitch + n0) = o;
            } else {
                *reinterpret_cast<float4*>(otile + m * p.opitch + n0) = make_float4(y[0], y[1], y[2], y[3]);
            }
        }
    }
    __syncthreads();
    const int nc = (p.N + V - 1) / V;
    for (int e = threadIdx.x; e < kRows * nc; e += kThreads) {
        const int r = e / nc, c = e % nc;
        const int64_t row = rows_of[r];
        if (row < 0) continue;
        float f[V];
        unpack<T>(*reinterpret_cast<const uint4*>(otile + r * p.opitch + c * V), f);
        const int n = min(V, p.N - c * V);
        if (p.pre) store_vals<T>(p.pre + row * p.ldy + c * V, f, n);
        if (p.relu) {
#pragma unroll
            for (int k = 0; k < V; ++k) f[k] = f[k] < 0.f ? 0.f : f[k];
        }
        store_vals<T>(p.Y + row * p.ldy + c * V, f, n);
    }
}

// Fragment-ordered W: entry (kg, nb, lane) holds the KG / 2 elements of
// column nb * 32 + lane % 32 at tile columns kg * KG + (KG / 2) (lane / 32)
// + q; tile column kk maps to W row kk (GCN), or kk (< d) and d + kk - koff
// (GraphSAGE, koff <= kk < koff + d); other columns are zero.
template <class T>
__global__ __launch_bounds__(256) void pack_fragments(const T* W, int64_t d, int64_t N, int koff, int self,
                                                      int kgroups, int NB, uint4* Bp) {
    constexpr int KG = kgroup<T>();
    const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (e >= static_cast<int64_t>(kgroups) * NB * 64) return;
    const int l = static_cast<int>(e % 64);
    const int nb = static_cast<int>((e / 64) % NB);
    const int kg = static_cast<int>(e / (64 * NB));
    const int64_t n = nb * 32 + (l & 31);
    uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < KG / 2; ++q) {
        const int64_t kk = static_cast<int64_t>(kg) * KG + (KG / 2) * (l >> 5) + q;
        int64_t wr = -1;
        if (self) {
            if (kk < d) wr = kk;
            else if (kk >= koff && kk < koff + d) wr = d + (kk - koff);
        } else if (kk < d) {
            wr = kk;
        }
        if (wr >= 0 && n < N) {
            if constexpr (sizeof(T) == 2)
                word[q / 2] |= static_cast<uint32_t>(W[wr * N + n]) << (16 * (q & 1));
            else
                word[q] = __float_as_uint(W[wr * N + n]);
        }
    }
    Bp[e] = make_uint4(word[0], word[1], word[2], word[3]);
}

struct Plan {
    int C = 0, koff = 0, kvalid = 0, kgroups = 0, NB = 0, pitch = 0, opitch = 0;
    size_t lds = 0;
};

Plan plan_of(int64_t d, int64_t N, bool self, sag_dtype dt) {
    Plan pl;
    const int V = static_cast<int>(vec_elems(dt));
    const int KG = dt == SAG_BF16 ? 16 : 8;
    const int es = static_cast<int>(elt_size(dt));
    pl.C = static_cast<int>(cdiv(d, V));
    pl.koff = self ? pl.C * V : 0;
    pl.kvalid = pl.koff + pl.C * V;
    pl.kgroups = static_cast<int>(cdiv(pl.kvalid, KG));
    pl.NB = static_cast<int>(cdiv(N, 32));
    // 16 bytes of padding per row spread the rows of an MFMA fragment read
    // over the LDS banks
    pl.pitch = pl.kgroups * KG + 16 / es;
    pl.opitch = pl.NB * 32 + 16 / es;
    pl.lds = static_cast<size_t>(std::max(kRows * pl.pitch, kRows * pl.opitch)) * es;
    return pl;
}

constexpr size_t kMaxLds = 96 * 1024;

}  // namespace

bool agg_transform_fits(int64_t d_in, int64_t d_out, bool self, sag_dtype dt) {
    if (d_in <= 0 || d_out <= 0 || d_out > kMaxNB * 32) return false;
    if (d_in > (dt == SAG_BF16 ? 2048 : 1024)) return false;
    return plan_of(d_in, d_out, self, dt).lds <= kMaxLds;
}

size_t agg_transform_ws_bytes(const sag_csr& A, int64_t d_in, int64_t d_out, bool self, sag_dtype dt) {
    const Plan pl = plan_of(d_in, d_out, self, dt);
    Carver c(nullptr, 0);
    c.take<uint4>(static_cast<size_t>(pl.kgroups) * pl.NB * 64);
    if (A.sched && A.n_long > 0) {
        c.take<char>(dense_bytes(A.n_long, d_in, dt));
        c.take<char>(spmm_long_ws_bytes(A, d_in));
    }
    return c.used();
}

namespace {

template <class T, int G, int NV>
void launch_at(const FusedArgs<T>& p, size_t lds, hipStream_t s) {
    // (once per kernel instance; thread-safe static initialisation)
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&agg_transform<T, G, NV>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(kMaxLds));
    (void)attr;
    agg_transform<T, G, NV><<<dim3(static_cast<unsigned>(p.n_tiles)), kThreads, lds, s>>>(p);
}

template <class T>
sag_status run_typed(const sag_csr& A, const void* H_ext, int64_t ldh, int64_t d_in, const void* W, const float* b,
                     int64_t d_out, bool self, int relu, sag_dtype dt, void* Y_pre, void* Out, int64_t ldo, void* Z,
                     int64_t ldz, void* ws, size_t ws_bytes, hipStream_t s) {
    const Plan pl = plan_of(d_in, d_out, self, dt);
    Carver c(ws, ws_bytes);
    uint4* Bp = c.take<uint4>(static_cast<size_t>(pl.kgroups) * pl.NB * 64);
    const bool has_long = A.sched && A.n_long > 0;
    void* zl = nullptr;
    void* sws = nullptr;
    size_t sws_bytes = 0;
    const int64_t ldzl = ldv(d_in, dt);
    if (has_long) {
        zl = c.take<char>(dense_bytes(A.n_long, d_in, dt));
        sws_bytes = spmm_long_ws_bytes(A, d_in);
        sws = c.take<char>(sws_bytes);
    }
    if (!c.fits()) return fail(SAG_E_WORKSPACE, "aggregate_transform: workspace too small");
    const int64_t nfrag = static_cast<int64_t>(pl.kgroups) * pl.NB * 64;
    pack_fragments<T><<<dim3(static_cast<unsigned>(cdiv(nfrag, 256))), 256, 0, s>>>(
        static_cast<const T*>(W), d_in, d_out, pl.koff, self ? 1 : 0, pl.kgroups, pl.NB, Bp);
    SAG_LAUNCH_CHECK();
    if (has_long) SAG_TRY(spmm_long_run(A, H_ext, ldh, dt, d_in, zl, ldzl, sws, sws_bytes, s));
    if (A.n_rows == 0) return SAG_OK;
    FusedArgs<T> p{};
    p.indptr = A.indptr;
    p.idx = A.indices;
    p.row_mean = A.row_mean != 0;
    p.val = p.row_mean ? nullptr : A.values;
    p.rec = reinterpret_cast<const int4*>(A.sched);
    p.n_rows = A.n_rows;
    p.n_summed = has_long ? A.n_short + A.n_medium : A.n_rows;
    p.X = static_cast<const T*>(H_ext);
    p.ldx = ldh;
    p.C = pl.C;
    p.d = static_cast<int>(d_in);
    p.self = self ? static_cast<const T*>(H_ext) : nullptr;
    p.ldself = ldh;
    p.zlong = static_cast<const T*>(zl);
    p.ldzl = ldzl;
    p.Z = static_cast<T*>(Z);
    p.ldz = ldz;
    p.Bp = Bp;
    p.kgroups = pl.kgroups;
    p.NB = pl.NB;
    p.koff = pl.koff;
    p.kvalid = pl.kvalid;
    p.pitch = pl.pitch;
    p.opitch = pl.opitch;
    p.N = static_cast<int>(d_out);
    p.bias = b;
    p.relu = relu;
    p.Y = static_cast<T*>(Out);
    p.pre = static_cast<T*>(Y_pre);
    p.ldy = ldo;
    p.n_tiles = cdiv(A.n_rows, kRows);
    p.n_short = A.sched ? A.n_short : 0;
    const int C = pl.C;
    if (C <= 4) launch_at<T, 4, 1>(p, pl.lds, s);
    else if (C <= 8) launch_at<T, 8, 1>(p, pl.lds, s);
    else if (C <= 16) launch_at<T, 16, 1>(p, pl.lds, s);
    else if (C <= 32) launch_at<T, 32, 1>(p, pl.lds, s);
    else if (C <= 64) launch_at<T, 64, 1>(p, pl.lds, s);
    else if (C <= 128) launch_at<T, 64, 2>(p, pl.lds, s);
    else if (C <= 192) launch_at<T, 64, 3>(p, pl.lds, s);
    else launch_at<T, 64, 4>(p, pl.lds, s);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace

sag_status agg_transform_run(const sag_csr& A, const void* H_ext, int64_t ldh, int64_t d_in, const void* W,
                             const float* b, int64_t d_out, bool self, int relu, sag_dtype dt, void* Y_pre, void* Out,
                             int64_t ldo, void* Z, int64_t ldz, void* ws, size_t ws_bytes, hipStream_t s) {
    const int64_t es = elt_size(dt);
    const int64_t K = (self ? 2 : 1) * d_in;
    // algorithmic bytes: CSR arrays, H_ext once, W, Z and the outputs once
    const int64_t bytes = 8 * (A.n_rows + 1) + A.nnz * (A.values && !A.row_mean ? 8 : 4) + es * d_in * A.n_cols +
                          es * K * d_out + (Z ? es * d_in * A.n_rows : 0) +
                          es * d_out * A.n_rows * (Y_pre ? 2 : 1);
    TraceScope trace(trace_enabled() ? shape_name(self ? "agg_transform_sage" : "agg_transform_gcn",
                                                  dt == SAG_BF16 ? "bf16" : "f32", A.n_rows, d_in, d_out)
                                     : std::string(),
                     s, bytes, 2 * A.nnz * d_in + 2 * A.n_rows * K * d_out);
    if (dt == SAG_BF16)
        return run_typed<uint16_t>(A, H_ext, ldh, d_in, W, b, d_out, self, relu, dt, Y_pre, Out, ldo, Z, ldz, ws,
                                   ws_bytes, s);
    return run_typed<float>(A, H_ext, ldh, d_in, W, b, d_out, self, relu, dt, Y_pre, Out, ldo, Z, ldz, ws, ws_bytes,
                            s);
}

}  // namespace sag

using namespace sag;

extern "C" size_t sag_aggregate_transform_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t d_out, int self,
                                                          sag_dtype dt) {
    if (!A || d_in <= 0 || d_out <= 0 || (dt != SAG_F32 && dt != SAG_BF16)) return 0;
    return agg_transform_ws_bytes(*A, d_in, d_out, self != 0, dt);
}

extern "C" sag_status sag_aggregate_transform(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                              const void* W, const float* b, int64_t d_out, int self, int relu,
                                              sag_dtype dt, void* Y_pre, void* Out, int64_t ldo, void* Z,
                                              int64_t ldz, void* ws, size_t ws_bytes, void* stream) {
    SAG_TRY(check_csr("aggregate_transform", A));
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "aggregate_transform: bad dtype");
    if (d_in <= 0 || d_out <= 0) return fail(SAG_E_INVALID, "aggregate_transform: widths must be positive");
    if (!agg_transform_fits(d_in, d_out, self != 0, dt))
        return fail(SAG_E_UNSUPPORTED, "aggregate_transform: d_out above 256 or the tile above the LDS budget");
    if (self && A->n_cols < A->n_rows)
        return fail(SAG_E_INVALID, "aggregate_transform: fewer columns than local rows");
    if (!W) return fail(SAG_E_INVALID, "aggregate_transform: null W");
    SAG_TRY(check_dense("aggregate_transform H_ext", H_ext, A->n_cols, d_in, ldh, dt));
    SAG_TRY(check_dense("aggregate_transform Out", Out, A->n_rows, d_out, ldo, dt));
    if (Y_pre) SAG_TRY(check_dense("aggregate_transform Y_pre", Y_pre, A->n_rows, d_out, ldo, dt));
    if (Z) SAG_TRY(check_dense("aggregate_transform Z", Z, A->n_rows, d_in, ldz, dt));
    if (ws_bytes < agg_transform_ws_bytes(*A, d_in, d_out, self != 0, dt) || !ws)
        return fail(SAG_E_WORKSPACE, "aggregate_transform: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "aggregate_transform: workspace not 16-B aligned");
    return agg_transform_run(*A, H_ext, ldh, d_in, W, b, d_out, self != 0, relu, dt, Y_pre, Out, ldo, Z, ldz, ws,
                             ws_bytes, static_cast<hipStream_t>(stream));
}


