// Graph-attention (GAT) layer on one partition, forward and backward.
//
// The pages name GAT (Velickovic et al., 2018) among the models that
// partitioned full-graph training serves (Sylvie, first section; DIGEST,
// evaluation section) without printing its formulas; the layer is the
// textbook one, with the heads side by side (head k owns columns
// [k d_head, (k + 1) d_head)):
//   Wh = H_ext W;  el[u] = a_src_k . Wh_k[u];  er[v] = a_dst_k . Wh_k[v];
//   x_vu = er[v] + el[u];  e_vu = LeakyReLU(x_vu) = lambda_vu x_vu
//   (lambda = 1 where x > 0, else the negative slope);
//   alpha_vu = exp(e_vu - lse[v]) with lse[v] = log sum_u exp(e_vu);
//   Out_k[v] = act(sum_u alpha_vu Wh_k[u] + b).
// Backward, with G_Y = G_out * 1[Y > 0] and, per head, dot_vu = G_Y[v] . Wh[u]:
//   c[v] = sum_u alpha_vu dot_vu;  ds_vu = alpha_vu (dot_vu - c[v]) lambda_vu;
//   der[v] = sum_u ds_vu = P[v] - c[v] Q[v] with P = sum alpha lambda dot and
//   Q = sum alpha lambda, so one sweep over row v gives it;
//   del[u] = sum_v ds_vu;  dWh[u] = sum_v alpha_vu G_Y[v] + del[u] a_src +
//   [u local] der[u] a_dst;  dW = H_ext^T dWh;  dH_ext = dWh W^T;
//   da_src = sum_u del[u] Wh[u];  da_dst = sum_v der[v] Wh[v];  db = colsum G_Y.
//
// No per-entry array is ever stored: the backward sweeps recompute alpha_vu
// from el, er and lse (12 bytes per row and head) instead of keeping
// nnz * heads floats.  Three sweeps over the entries share the SpMM's
// degree-binned schedule and its lane layout (a group of G lanes covers one
// 16-byte-vector row; short rows one group each, medium rows one wavefront,
// long rows cut into segments whose fp32 partials a second kernel combines
// in order):
//   fwd  over A  : Out and lse, gathering rows of Wh, with the softmax taken
//                  online (a running max m, the sum s of exp(e - m) and the
//                  accumulator, rescaled when m grows; partial states merge
//                  by rescaling to the larger max), so no separate pass
//                  computes the normalisers;
//   bwa  over A  : c and der, gathering rows of Wh against the row's own G_Y;
//   bwt  over AT : dWh and del of each row u of [local | halo], gathering
//                  rows of G_Y and one 16-byte record {er, lse, c} per head.
// fwd and bwa take el[u] of a gathered row from the row itself (its dot
// product with a_src, computed exactly as the score kernel does), so an
// entry costs the row's cache lines and nothing more.
// Each lane owns the heads of its vectors; the per-entry dot products are
// finished with a butterfly over the d_head / V lanes of a head.
#include <algorithm>
#include <cmath>

#include "ops.h"
#include "trace.h"

namespace sag {
namespace {

constexpr int kWaves = 4;
enum { M_FWD = 1, M_BWA = 2, M_BWT = 3 };

struct GatArgs {
    const int64_t* indptr;
    const int32_t* idx;
    const int4* rec_short;
    const int4* rec_medium;   // null: every row is medium, natural order
    const int4* rec_long;
    const int4* seg;
    const int32_t* seg0;
    int64_t n_short, n_medium, n_long, n_seg;
    int64_t nb_seg, nb_medium;
    int C;          // 16-byte vectors per row
    int H;          // heads
    int hshift;     // log2(vectors per head)
    float slope;
    const void* X;  // gathered rows: Wh (fwd, bwa) or G_Y (bwt)
    int64_t ldx;
    const void* own;   // the row's own vector: G_out (bwa) or Wh (bwt)
    int64_t ldown;
    const void* ymask; // bwa: Y, whose sign masks G_out (null: no ReLU)
    int64_t ldym;
    void* gy;          // bwa: G_Y written here (nullable)
    int64_t ldgy;
    const float* el;
    const float* er;
    const float* lse;
    const float4* rinfo;   // bwt: {er, lse, c, 0} per (local row, head)
    const float* der;      // bwt: der per (local row, head)
    float* o_lse;
    float4* o_rinfo;
    float* o_der;
    float* o_del;
    void* y;               // fwd: Out; bwt: dWh
    int64_t ldy;
    const float* bias;
    int relu;
    const float* a_src;
    const float* a_dst;
    int64_t n_local;
    float* part;           // segment partials, ldp floats each
    int ldp;
    int soff;              // offset of the per-head statistics in a partial
};

__device__ __forceinline__ int64_t rec_start(const int4& r) {
    return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(r.z)) |
                                (static_cast<uint64_t>(static_cast<uint32_t>(r.w)) << 32));
}

template <class T>
__device__ __forceinline__ uint4 load_row_vec(const T* X, int64_t ld, int64_t r, int ch) {
    return *reinterpret_cast<const uint4*>(X + r * ld + ch * Vec<T>::N);
}

// exp(a - b) for a running max b >= a; an empty side (a = -inf) gives 0.
__device__ __forceinline__ float rescale(float a, float b) { return a == -INFINITY ? 0.f : __expf(a - b); }

// Per-lane state of one row sweep.
template <int MODE, class T, int NV>
struct Lane {
    static constexpr int V = Vec<T>::N;
    int ch[NV];        // vector index (clamped to the row)
    int hd[NV];        // head of that vector
    float acc[NV][V];  // fwd, bwt
    float own[NV][V];  // bwa: G_Y[v]; bwt: Wh[u]
    float r0[NV], r1[NV];       // fwd: er; bwa: er, lse; bwt: el
    float s0[NV], s1[NV], s2[NV];  // fwd: running max, sum; bwa: c, P, Q; bwt: del
    float as[NV][V];   // fwd, bwa: a_src over the vector's elements
};

template <int MODE, class T, int NV>
__device__ __forceinline__ void lane_init(Lane<MODE, T, NV>& L, const GatArgs& p, int gl, int G) {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        L.ch[v] = min(v * G + gl, p.C - 1);
        L.hd[v] = L.ch[v] >> p.hshift;
        L.r0[v] = L.r1[v] = 0.f;
        L.s0[v] = MODE == M_FWD ? -INFINITY : 0.f;
        L.s1[v] = L.s2[v] = 0.f;
#pragma unroll
        for (int k = 0; k < Lane<MODE, T, NV>::V; ++k) {
            L.acc[v][k] = L.own[v][k] = 0.f;
            L.as[v][k] = MODE == M_BWT ? 0.f : p.a_src[L.ch[v] * Lane<MODE, T, NV>::V + k];
        }
    }
}

// The row's own values; `write_gy` stores G_Y (bwa with a mask).
template <int MODE, class T, int NV>
__device__ __forceinline__ void lane_row(Lane<MODE, T, NV>& L, const GatArgs& p, int64_t row, bool write_gy) {
    constexpr int V = Vec<T>::N;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int64_t rh = row * p.H + L.hd[v];
        if constexpr (MODE == M_FWD) {
            L.r0[v] = p.er[rh];
        } else if constexpr (MODE == M_BWA) {
            L.r0[v] = p.er[rh];
            L.r1[v] = p.lse[rh];
        } else {
            L.r0[v] = p.el[rh];
        }
        if constexpr (MODE == M_BWA || MODE == M_BWT) {
            const T* o = static_cast<const T*>(p.own);
            unpack<T>(load_row_vec(o, p.ldown, row, L.ch[v]), L.own[v]);
        }
        if constexpr (MODE == M_BWA) {
            if (p.ymask) {
                float ym[V];
                unpack<T>(load_row_vec(static_cast<const T*>(p.ymask), p.ldym, row, L.ch[v]), ym);
#pragma unroll
                for (int k = 0; k < V; ++k) L.own[v][k] = ym[k] > 0.f ? L.own[v][k] : 0.f;
                if (write_gy)
                    store_vals<T>(static_cast<T*>(p.gy) + row * p.ldgy + L.ch[v] * V, L.own[v], V);
            }
        }
    }
}

// x plus its value in another lane through a DPP lane permutation (one
// VALU instruction, no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum of a value over the lanes of one head (2^hshift consecutive lanes,
// aligned): swaps within quads (lanes 1 and 2 apart), then mirrors within 8
// and 16 lanes -- after each step every lane of the group holds the group's
// sum, so a mirror adds the other half's sum -- then lane shuffles for 32
// and 64.
__device__ __forceinline__ float head_sum(float x, int hshift) {
    if (hshift >= 1) x = dpp_add<0xb1>(x);    // quad_perm [1, 0, 3, 2]
    if (hshift >= 2) x = dpp_add<0x4e>(x);    // quad_perm [2, 3, 0, 1]
    if (hshift >= 3) x = dpp_add<0x141>(x);   // row_half_mirror
    if (hshift >= 4) x = dpp_add<0x140>(x);   // row_mirror
    if (hshift >= 5) x += __shfl_xor(x, 16, 64);
    if (hshift >= 6) x += __shfl_xor(x, 32, 64);
    return x;
}

// U entries (columns c[u], live where ok[u]) into the lane state.
template <int MODE, class T, int NV, int U>
__device__ __forceinline__ void lane_entries(Lane<MODE, T, NV>& L, const GatArgs& p, const int32_t (&c)[U],
                                             const bool (&ok)[U]) {
    constexpr int V = Vec<T>::N;
    const T* X = static_cast<const T*>(p.X);
    uint4 x[U][NV];
    float sc[U][NV];
    float4 ri[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            x[u][v] = load_row_vec(X, p.ldx, c[u], L.ch[v]);
            if constexpr (MODE == M_BWT) ri[u][v] = p.rinfo[static_cast<int64_t>(c[u]) * p.H + L.hd[v]];
        }
    if constexpr (MODE != M_BWT) {
        // el of each gathered row, recomputed from the row itself rather than
        // gathered (one cache line less per entry): the same products, order
        // and butterfly as the score kernel, so the same bits
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                float f[V];
                unpack<T>(x[u][v], f);
                float ps = 0.f;
#pragma unroll
                for (int k = 0; k < V; ++k) ps = fmaf(f[k], L.as[v][k], ps);
                sc[u][v] = head_sum(ps, p.hshift);
            }
    }
    if constexpr (MODE == M_FWD) {
        // the batch's scores, one rescale of the state to the new max, then
        // the entries' terms
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float ev[U];
            float bm = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float xx = L.r0[v] + sc[u][v];
                ev[u] = ok[u] ? xx * (xx > 0.f ? 1.f : p.slope) : -INFINITY;
                bm = fmaxf(bm, ev[u]);
            }
            const float mn = fmaxf(L.s0[v], bm);
            if (mn != -INFINITY) {
                const float f = rescale(L.s0[v], mn);
                L.s1[v] *= f;
#pragma unroll
                for (int k = 0; k < V; ++k) L.acc[v][k] *= f;
                L.s0[v] = mn;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const float a = rescale(ev[u], mn);
                    float f2[V];
                    unpack<T>(x[u][v], f2);
                    L.s1[v] += a;
                    // (a select, not a zero weight: a dead entry reads row 0,
                    // whatever it holds)
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const float t2 = fmaf(a, f2[k], L.acc[v][k]);
                        L.acc[v][k] = ok[u] ? t2 : L.acc[v][k];
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float f[V];
            unpack<T>(x[u][v], f);
            {
                float part = 0.f;
#pragma unroll
                for (int k = 0; k < V; ++k) part = fmaf(L.own[v][k], f[k], part);
                const float dot = head_sum(part, p.hshift);
                if constexpr (MODE == M_BWA) {
                    const float xx = L.r0[v] + sc[u][v];
                    const float lam = xx > 0.f ? 1.f : p.slope;
                    const float a = ok[u] ? __expf(xx * lam - L.r1[v]) : 0.f;
                    const float al = a * lam;
                    // (selects: a dead entry reads row 0, whatever it holds)
                    L.s0[v] = ok[u] ? fmaf(a, dot, L.s0[v]) : L.s0[v];
                    L.s1[v] = ok[u] ? fmaf(al, dot, L.s1[v]) : L.s1[v];
                    L.s2[v] += al;
                } else {
                    const float xx = ri[u][v].x + L.r0[v];
                    const float lam = xx > 0.f ? 1.f : p.slope;
                    const float a = ok[u] ? __expf(xx * lam - ri[u][v].y) : 0.f;
                    L.s0[v] = ok[u] ? fmaf(a * lam, dot - ri[u][v].z, L.s0[v]) : L.s0[v];
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const float t2 = fmaf(a, f[k], L.acc[v][k]);
                        L.acc[v][k] = ok[u] ? t2 : L.acc[v][k];
                    }
                }
            }
        }
    }
}

template <int NV>
constexpr int unroll_of() { return NV >= 4 ? 2 : (NV >= 2 ? 4 : 8); }

// Entries [start, start + len) of one row for a group of G lanes (short
// rows: P rows per wavefront, lmax the wavefront's longest).
template <int MODE, class T, int G, int NV>
__device__ __forceinline__ void sweep_group(Lane<MODE, T, NV>& L, const GatArgs& p, int64_t start, int len,
                                            int lmax) {
    constexpr int U = unroll_of<NV>();
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    for (int j0 = 0; j0 < lmax; j0 += G) {
        const int jj = j0 + gl;
        const int32_t c_my = jj < len ? p.idx[start + jj] : 0;
        const int nh = min(G, lmax - j0);
        for (int t = 0; t < nh; t += U) {
            int32_t c[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                c[u] = __shfl(c_my, grp * G + min(t + u, G - 1), 64);
                ok[u] = (t + u < nh) && (j0 + t + u < len);
            }
            lane_entries<MODE, T, NV, U>(L, p, c, ok);
        }
    }
}

// Entries of one row for the whole wavefront: group g takes entries g,
// g + P, ...; the group states are then combined by a fixed butterfly.
template <int MODE, class T, int G, int NV>
__device__ __forceinline__ void sweep_wave(Lane<MODE, T, NV>& L, const GatArgs& p, int64_t start, int len) {
    constexpr int U = unroll_of<NV>();
    constexpr int P = 64 / G;
    constexpr int V = Vec<T>::N;
    const int lane = threadIdx.x & 63;
    const int grp = lane / G;
    for (int j0 = 0; j0 < len; j0 += 64) {
        const int jj = j0 + lane;
        const int32_t c_my = jj < len ? p.idx[start + jj] : 0;
        const int nh = min(64, len - j0);
        for (int t = 0; t < nh; t += U * P) {
            int32_t c[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int src = t + u * P + grp;
                c[u] = __shfl(c_my, min(src, 63), 64);
                ok[u] = src < nh;
            }
            lane_entries<MODE, T, NV, U>(L, p, c, ok);
        }
    }
#pragma unroll
    for (int off = G; off < 64; off <<= 1) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if constexpr (MODE == M_FWD) {
                const float m2 = __shfl_xor(L.s0[v], off, 64), s2 = __shfl_xor(L.s1[v], off, 64);
                const float mn = fmaxf(L.s0[v], m2);
                const float f1 = rescale(L.s0[v], mn), f2 = rescale(m2, mn);
                L.s1[v] = L.s1[v] * f1 + s2 * f2;
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float o = __shfl_xor(L.acc[v][k], off, 64);
                    L.acc[v][k] = L.acc[v][k] * f1 + o * f2;
                }
                L.s0[v] = mn;
            } else {
                if constexpr (MODE == M_BWT) {
#pragma unroll
                    for (int k = 0; k < V; ++k) L.acc[v][k] += __shfl_xor(L.acc[v][k], off, 64);
                }
                if constexpr (MODE == M_BWA || MODE == M_BWT) L.s0[v] += __shfl_xor(L.s0[v], off, 64);
                if constexpr (MODE == M_BWA) {
                    L.s1[v] += __shfl_xor(L.s1[v], off, 64);
                    L.s2[v] += __shfl_xor(L.s2[v], off, 64);
                }
            }
        }
    }
}

// Outputs of one row from a combined lane state, for vector v of the lane
// (cv = its unclamped index).
template <int MODE, class T, int NV>
__device__ __forceinline__ void row_out(const Lane<MODE, T, NV>& L, const GatArgs& p, const float* cvec, int64_t row,
                                        int v, int cv) {
    constexpr int V = Vec<T>::N;
    if (cv >= p.C) return;
    const int hd = L.hd[v];
    const int64_t rh = row * p.H + hd;
    const bool head_lead = (cv & ((1 << p.hshift) - 1)) == 0;
    if constexpr (MODE == M_FWD) {
        const float s = L.s1[v];
        const float inv = s > 0.f ? 1.f / s : 0.f;
        float a[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
            float t = L.acc[v][k] * inv;
            if (p.bias) t += cvec[cv * V + k];
            a[k] = p.relu && t < 0.f ? 0.f : t;
        }
        store_vals<T>(static_cast<T*>(p.y) + row * p.ldy + cv * V, a, V);
        if (head_lead) p.o_lse[rh] = s > 0.f ? L.s0[v] + __logf(s) : -INFINITY;
    } else if constexpr (MODE == M_BWA) {
        if (head_lead) {
            p.o_rinfo[rh] = make_float4(L.r0[v], L.r1[v], L.s0[v], 0.f);
            p.o_der[rh] = L.s1[v] - L.s0[v] * L.s2[v];
        }
    } else {
        const float dl = L.s0[v];
        const float dr = row < p.n_local ? p.der[rh] : 0.f;
        float a[V];
#pragma unroll
        for (int k = 0; k < V; ++k)
            a[k] = L.acc[v][k] + dl * p.a_src[cv * V + k] + dr * p.a_dst[cv * V + k];
        store_vals<T>(static_cast<T*>(p.y) + row * p.ldy + cv * V, a, V);
        if (head_lead) p.o_del[rh] = dl;
    }
}

template <int MODE, class T, int G, int NV>
__device__ __forceinline__ void short_rows(const GatArgs& p, const float* cvec, int64_t block) {
    constexpr int P = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    const int64_t i = (block * kWaves + (threadIdx.x >> 6)) * P + grp;
    const bool valid = i < p.n_short;
    int64_t row = 0, start = 0;
    int len = 0;
    if (valid) {
        const int4 r = p.rec_short[i];
        row = r.x;
        len = r.y;
        start = rec_start(r);
    }
    int lmax = len;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lmax = max(lmax, __shfl_xor(lmax, off, 64));
    Lane<MODE, T, NV> L;
    lane_init(L, p, gl, G);
    if (valid) lane_row(L, p, row, true);
    sweep_group<MODE, T, G, NV>(L, p, start, len, lmax);
    if (!valid) return;
#pragma unroll
    for (int v = 0; v < NV; ++v) row_out(L, p, cvec, row, v, v * G + gl);
}

template <int MODE, class T, int G, int NV>
__device__ __forceinline__ void medium_rows(const GatArgs& p, const float* cvec, int64_t block) {
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
    const int gl = lane % G;
    Lane<MODE, T, NV> L;
    lane_init(L, p, gl, G);
    lane_row(L, p, row, lane < G);
    sweep_wave<MODE, T, G, NV>(L, p, start, len);
    if (lane >= G) return;
#pragma unroll
    for (int v = 0; v < NV; ++v) row_out(L, p, cvec, row, v, v * G + gl);
}

template <int MODE, class T, int G, int NV>
__device__ __forceinline__ void segments(const GatArgs& p, int64_t block) {
    constexpr int V = Vec<T>::N;
    const int64_t sidx = block * kWaves + (threadIdx.x >> 6);
    if (sidx >= p.n_seg) return;
    const int4 sr = p.seg[sidx];
    const int64_t start = static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(sr.y)) |
                                               (static_cast<uint64_t>(static_cast<uint32_t>(sr.z)) << 32));
    const int64_t row = p.rec_long[sr.x].x;
    const int lane = threadIdx.x & 63;
    const int gl = lane % G;
    Lane<MODE, T, NV> L;
    lane_init(L, p, gl, G);
    lane_row(L, p, row, false);
    sweep_wave<MODE, T, G, NV>(L, p, start, sr.w);
    if (lane >= G) return;
    float* out = p.part + sidx * static_cast<int64_t>(p.ldp);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int cv = v * G + gl;
        if (cv >= p.C) continue;
        if constexpr (MODE == M_FWD || MODE == M_BWT) {
#pragma unroll
            for (int q = 0; q < V; q += 4)
                *reinterpret_cast<float4*>(out + cv * V + q) =
                    make_float4(L.acc[v][q], L.acc[v][q + 1], L.acc[v][q + 2], L.acc[v][q + 3]);
        }
        if ((cv & ((1 << p.hshift) - 1)) == 0) {
            float* st = out + p.soff + L.hd[v] * 3;
            st[0] = L.s0[v];
            st[1] = L.s1[v];
            st[2] = L.s2[v];
        }
    }
}

// The forward's bias (zeros without one) copied to LDS once per workgroup:
// read from global memory at the end of every row it costs a memory round
// trip per row, and kept in registers it would cost occupancy.  (The column
// sweep's a_src and a_dst measured no faster this way.)
template <int MODE, class T>
__device__ __forceinline__ void load_cvec(const GatArgs& p, float* cvec) {
    constexpr int V = Vec<T>::N;
    const int F = p.C * V;
    for (int i = threadIdx.x; i < F; i += blockDim.x) cvec[i] = p.bias ? p.bias[i] : 0.f;
    __syncthreads();
}

template <int MODE>
constexpr int cvec_count() { return MODE == M_FWD ? 1 : 0; }

template <int MODE, class T, int G, int NV>
__global__ __launch_bounds__(256) void gat_bins(GatArgs p) {
    extern __shared__ float cvec[];
    if constexpr (cvec_count<MODE>() > 0) load_cvec<MODE, T>(p, cvec);
    int64_t b = blockIdx.x;
    if (b < p.nb_seg) {
        segments<MODE, T, G, NV>(p, b);
        return;
    }
    b -= p.nb_seg;
    if (b < p.nb_medium) {
        medium_rows<MODE, T, G, NV>(p, cvec, b);
        return;
    }
    short_rows<MODE, T, G, NV>(p, cvec, b - p.nb_medium);
}

// Combines the segment partials of each long row in segment order, then
// the row's outputs (one wavefront per long row, lanes over vectors).
template <int MODE, class T>
__global__ __launch_bounds__(256) void gat_long_reduce(GatArgs p) {
    constexpr int V = Vec<T>::N;
    extern __shared__ float cvec[];
    if constexpr (cvec_count<MODE>() > 0) load_cvec<MODE, T>(p, cvec);
    const int64_t j = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (j >= p.n_long) return;
    const int lane = threadIdx.x & 63;
    const int64_t row = p.rec_long[j].x;
    const int32_t s0 = p.seg0[j], s1 = p.seg0[j + 1];
    for (int cv = lane; cv < p.C; cv += 64) {
        Lane<MODE, T, 1> L;
        L.ch[0] = cv;
        L.hd[0] = cv >> p.hshift;
        L.s0[0] = MODE == M_FWD ? -INFINITY : 0.f;
        L.s1[0] = L.s2[0] = 0.f;
#pragma unroll
        for (int k = 0; k < V; ++k) L.acc[0][k] = 0.f;
        for (int32_t s = s0; s < s1; ++s) {
            const float* src = p.part + static_cast<int64_t>(s) * p.ldp;
            const float* st = src + p.soff + L.hd[0] * 3;
            float f1 = 1.f, f2 = 1.f;
            if constexpr (MODE == M_FWD) {
                const float mn = fmaxf(L.s0[0], st[0]);
                f1 = rescale(L.s0[0], mn);
                f2 = rescale(st[0], mn);
                L.s1[0] = L.s1[0] * f1 + st[1] * f2;
                L.s0[0] = mn;
            } else {
                L.s0[0] += st[0];
                L.s1[0] += st[1];
                L.s2[0] += st[2];
            }
            if constexpr (MODE == M_FWD || MODE == M_BWT) {
#pragma unroll
                for (int q = 0; q < V; q += 4) {
                    const float4 t = *reinterpret_cast<const float4*>(src + cv * V + q);
                    L.acc[0][q] = L.acc[0][q] * f1 + t.x * f2;
                    L.acc[0][q + 1] = L.acc[0][q + 1] * f1 + t.y * f2;
                    L.acc[0][q + 2] = L.acc[0][q + 2] * f1 + t.z * f2;
                    L.acc[0][q + 3] = L.acc[0][q + 3] * f1 + t.w * f2;
                }
            }
        }
        const int64_t rh = row * p.H + L.hd[0];
        if constexpr (MODE == M_BWA) {
            L.r0[0] = p.er[rh];
            L.r1[0] = p.lse[rh];
            if (p.ymask && p.gy) {
                float g[V], ym[V];
                unpack<T>(load_row_vec(static_cast<const T*>(p.own), p.ldown, row, cv), g);
                unpack<T>(load_row_vec(static_cast<const T*>(p.ymask), p.ldym, row, cv), ym);
#pragma unroll
                for (int k = 0; k < V; ++k) g[k] = ym[k] > 0.f ? g[k] : 0.f;
                store_vals<T>(static_cast<T*>(p.gy) + row * p.ldgy + cv * V, g, V);
            }
        }
        row_out(L, p, cvec, row, 0, cv);
    }
}

// el and er of every row of Wh: one group of G lanes per row.
template <class T, int G, int NV>
__global__ __launch_bounds__(256) void gat_scores(const T* Wh, int64_t ld, int64_t n, int C, int H, int hshift,
                                                  const float* a_src, const float* a_dst, float* el, float* er) {
    constexpr int V = Vec<T>::N;
    constexpr int P = 64 / G;
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    const int64_t r = (static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6)) * P + grp;
    const bool valid = r < n;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int cv = v * G + gl;
        const int ch = min(cv, C - 1);
        float f[V];
        if (valid) {
            unpack<T>(load_row_vec(Wh, ld, r, ch), f);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) f[k] = 0.f;
        }
        float ps = 0.f, pd = 0.f;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            ps = fmaf(f[k], a_src[ch * V + k], ps);
            pd = fmaf(f[k], a_dst[ch * V + k], pd);
        }
        ps = head_sum(ps, hshift);
        pd = head_sum(pd, hshift);
        if (valid && cv < C && (cv & ((1 << hshift) - 1)) == 0) {
            el[r * H + (cv >> hshift)] = ps;
            er[r * H + (cv >> hshift)] = pd;
        }
    }
}

// Weighted column sums, stage 1: part[b][j] = sum over block b's rows r of
// w[r, head(j)] X[r, j] (w null: weight 1), in a fixed order.
template <class T>
__global__ __launch_bounds__(256) void gat_colsum_part(const T* X, int64_t ldx, int64_t n, int C, int Cp, int H,
                                                       int hshift, const float* w, int64_t rows_per_block,
                                                       float* part) {
    constexpr int V = Vec<T>::N;
    __shared__ float red[256 * V];
    const int t = threadIdx.x;
    const int ch = t % Cp, rr = t / Cp, RP = 256 / Cp;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
    const int64_t r1 = min(n, r0 + rows_per_block);
    float a[V];
#pragma unroll
    for (int k = 0; k < V; ++k) a[k] = 0.f;
    if (ch < C) {
        for (int64_t r = r0 + rr; r < r1; r += RP) {
            float f[V];
            unpack<T>(load_row_vec(X, ldx, r, ch), f);
            const float wt = w ? w[r * H + (ch >> hshift)] : 1.f;
#pragma unroll
            for (int k = 0; k < V; ++k) a[k] = fmaf(wt, f[k], a[k]);
        }
    }
#pragma unroll
    for (int k = 0; k < V; ++k) red[t * V + k] = a[k];
    __syncthreads();
    const int F = C * V;
    for (int j = t; j < F; j += 256) {
        float s = 0.f;
        for (int q = 0; q < RP; ++q) s += red[q * Cp * V + j];
        part[static_cast<int64_t>(blockIdx.x) * F + j] = s;
    }
}

// Stage 1 of two weighted column sums of the same X in one pass over its
// rows: part1 over rows [0, n1) with weights w1, part2 over rows [0, n2)
// with w2 (n1 <= n2), each block and each sum in the order of
// gat_colsum_part, so the results equal two separate passes.
template <class T>
__global__ __launch_bounds__(256) void gat_colsum2_part(const T* X, int64_t ldx, int64_t n1, int64_t n2, int C,
                                                        int Cp, int H, int hshift, const float* w1,
                                                        const float* w2, int64_t rows_per_block, int64_t nb1,
                                                        float* part1, float* part2) {
    constexpr int V = Vec<T>::N;
    __shared__ float red[2][256 * V];
    const int t = threadIdx.x;
    const int ch = t % Cp, rr = t / Cp, RP = 256 / Cp;
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_block;
    const int64_t r1 = min(n2, r0 + rows_per_block), r1a = min(n1, r0 + rows_per_block);
    float a[V], b[V];
#pragma unroll
    for (int k = 0; k < V; ++k) a[k] = b[k] = 0.f;
    if (ch < C) {
        for (int64_t r = r0 + rr; r < r1; r += RP) {
            float f[V];
            unpack<T>(load_row_vec(X, ldx, r, ch), f);
            const int64_t rh = r * H + (ch >> hshift);
            const float wb = w2[rh];
#pragma unroll
            for (int k = 0; k < V; ++k) b[k] = fmaf(wb, f[k], b[k]);
            if (r < r1a) {
                const float wa = w1[rh];
#pragma unroll
                for (int k = 0; k < V; ++k) a[k] = fmaf(wa, f[k], a[k]);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
        red[0][t * V + k] = a[k];
        red[1][t * V + k] = b[k];
    }
    __syncthreads();
    const int F = C * V;
    for (int j = t; j < F; j += 256) {
        float sa = 0.f, sb = 0.f;
        for (int q = 0; q < RP; ++q) {
            sa += red[0][q * Cp * V + j];
            sb += red[1][q * Cp * V + j];
        }
        if (blockIdx.x < nb1) part1[static_cast<int64_t>(blockIdx.x) * F + j] = sa;
        part2[static_cast<int64_t>(blockIdx.x) * F + j] = sb;
    }
}

// Stage 2: out[j] = sum over blocks of part[b][j], blocks in order; 64
// columns per workgroup, four interleaved block ranges added at the end.
__global__ __launch_bounds__(256) void gat_colsum_final(const float* part, int64_t nb, int F, float* out) {
    __shared__ float red[256];
    const int jj = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + jj;
    float s = 0.f;
    if (j < F)
        for (int64_t b = q; b < nb; b += 4) s += part[b * F + j];
    red[threadIdx.x] = s;
    __syncthreads();
    if (q == 0 && j < F) out[j] = ((red[jj] + red[64 + jj]) + red[128 + jj]) + red[192 + jj];
}

// ---- host side ------------------------------------------------------------------------

struct Heads {
    int64_t H = 0, dh = 0, F = 0;
    int C = 0, hshift = 0;
};

sag_status heads_of(const char* who, int64_t heads, int64_t d_head, sag_dtype dt, Heads* h) {
    const std::string w(who);
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, w + ": bad dtype");
    if (heads < 1 || d_head < 1) return fail(SAG_E_INVALID, w + ": heads and d_head must be positive");
    const int64_t V = vec_elems(dt);
    const int64_t ch = d_head / V;
    if (d_head % V != 0 || (ch & (ch - 1)) != 0 || ch > 64)
        return fail(SAG_E_UNSUPPORTED, w + ": d_head must be a power-of-two number of 16-byte vectors, at most 64");
    if (heads > 64) return fail(SAG_E_UNSUPPORTED, w + ": at most 64 heads");
    const int64_t F = heads * d_head;
    if (F > (dt == SAG_BF16 ? 2048 : 1024)) return fail(SAG_E_UNSUPPORTED, w + ": heads * d_head too large");
    h->H = heads;
    h->dh = d_head;
    h->F = F;
    h->C = static_cast<int>(F / V);
    int s = 0;
    while ((int64_t(1) << s) < ch) ++s;
    h->hshift = s;
    return SAG_OK;
}

void set_sched(const sag_csr& A, GatArgs& p) {
    p.indptr = A.indptr;
    p.idx = A.indices;
    const int4* rec = reinterpret_cast<const int4*>(A.sched);
    p.rec_short = p.rec_medium = p.rec_long = p.seg = nullptr;
    p.seg0 = nullptr;
    p.n_short = p.n_long = p.n_seg = 0;
    if (!rec) {
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
}

int64_t seg_count(const sag_csr& A) { return (A.sched && A.n_long > 0) ? A.n_seg : 0; }

// Floats per segment partial: C * V accumulators, then 3 per head.
int partial_floats(const Heads& h, sag_dtype dt) {
    return static_cast<int>(round_up(h.C * vec_elems(dt) + 3 * h.H, 4));
}

template <int MODE, class T, int G, int NV>
sag_status launch_g(GatArgs p, hipStream_t s) {
    constexpr int P = 64 / G;
    p.nb_seg = cdiv(p.n_seg, kWaves);
    p.nb_medium = cdiv(p.n_medium, kWaves);
    const int64_t blocks = p.nb_seg + p.nb_medium + cdiv(p.n_short, kWaves * P);
    const size_t lds = static_cast<size_t>(cvec_count<MODE>()) * p.C * Vec<T>::N * sizeof(float);
    if (blocks > 0) {
        gat_bins<MODE, T, G, NV><<<dim3(static_cast<unsigned>(blocks)), 256, lds, s>>>(p);
        SAG_LAUNCH_CHECK();
    }
    if (p.n_long > 0) {
        gat_long_reduce<MODE, T><<<dim3(static_cast<unsigned>(cdiv(p.n_long, kWaves))), 256, lds, s>>>(p);
        SAG_LAUNCH_CHECK();
    }
    return SAG_OK;
}

template <int MODE, class T>
sag_status launch_pass(const sag_csr& A, GatArgs p, hipStream_t s) {
    set_sched(A, p);
    if (A.n_rows == 0) return SAG_OK;
    const int C = p.C;
    if (C <= 4) return launch_g<MODE, T, 4, 1>(p, s);
    if (C <= 8) return launch_g<MODE, T, 8, 1>(p, s);
    if (C <= 16) return launch_g<MODE, T, 16, 1>(p, s);
    if (C <= 32) return launch_g<MODE, T, 32, 1>(p, s);
    if (C <= 64) return launch_g<MODE, T, 64, 1>(p, s);
    if (C <= 128) return launch_g<MODE, T, 64, 2>(p, s);
    if (C <= 192) return launch_g<MODE, T, 64, 3>(p, s);
    if (C <= 256) return launch_g<MODE, T, 64, 4>(p, s);
    return fail(SAG_E_UNSUPPORTED, "gat: row too wide");
}

template <class T>
sag_status launch_scores(const Heads& h, const void* Wh, int64_t ld, int64_t n, const float* a_src,
                         const float* a_dst, float* el, float* er, hipStream_t s) {
    if (n == 0) return SAG_OK;
    const T* w = static_cast<const T*>(Wh);
    auto go = [&](auto g_tag, auto nv_tag) {
        constexpr int G = decltype(g_tag)::value, NV = decltype(nv_tag)::value;
        const int64_t blocks = cdiv(n, kWaves * (64 / G));
        gat_scores<T, G, NV><<<dim3(static_cast<unsigned>(blocks)), 256, 0, s>>>(w, ld, n, h.C, static_cast<int>(h.H),
                                                                               h.hshift, a_src, a_dst, el, er);
    };
    using std::integral_constant;
    const int C = h.C;
    if (C <= 4) go(integral_constant<int, 4>{}, integral_constant<int, 1>{});
    else if (C <= 8) go(integral_constant<int, 8>{}, integral_constant<int, 1>{});
    else if (C <= 16) go(integral_constant<int, 16>{}, integral_constant<int, 1>{});
    else if (C <= 32) go(integral_constant<int, 32>{}, integral_constant<int, 1>{});
    else if (C <= 64) go(integral_constant<int, 64>{}, integral_constant<int, 1>{});
    else if (C <= 128) go(integral_constant<int, 64>{}, integral_constant<int, 2>{});
    else if (C <= 192) go(integral_constant<int, 64>{}, integral_constant<int, 3>{});
    else go(integral_constant<int, 64>{}, integral_constant<int, 4>{});
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

constexpr int64_t kColsumRows = 2048;

int64_t colsum_blocks(int64_t n) { return n > 0 ? cdiv(n, kColsumRows) : 0; }

template <class T>
sag_status launch_colsum(const Heads& h, const void* X, int64_t ldx, int64_t n, const float* w, float* part,
                         float* out, hipStream_t s) {
    const int F = static_cast<int>(h.F);
    const int64_t nb = colsum_blocks(n);
    if (nb > 0) {
        int Cp = 1;
        while (Cp < h.C) Cp <<= 1;
        gat_colsum_part<T><<<dim3(static_cast<unsigned>(nb)), 256, 0, s>>>(
            static_cast<const T*>(X), ldx, n, h.C, Cp, static_cast<int>(h.H), h.hshift, w, kColsumRows, part);
        SAG_LAUNCH_CHECK();
    }
    gat_colsum_final<<<dim3(static_cast<unsigned>(cdiv(F, 64))), 256, 0, s>>>(part, nb, F, out);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

// da_dst (rows [0, n1), weights w1) and da_src (rows [0, n2), weights w2)
// from one pass over Wh.
template <class T>
sag_status launch_colsum2(const Heads& h, const void* X, int64_t ldx, int64_t n1, const float* w1, float* part1,
                          float* out1, int64_t n2, const float* w2, float* part2, float* out2, hipStream_t s) {
    const int F = static_cast<int>(h.F);
    const int64_t nb1 = colsum_blocks(n1), nb2 = colsum_blocks(n2);
    if (nb2 > 0) {
        int Cp = 1;
        while (Cp < h.C) Cp <<= 1;
        gat_colsum2_part<T><<<dim3(static_cast<unsigned>(nb2)), 256, 0, s>>>(
            static_cast<const T*>(X), ldx, n1, n2, h.C, Cp, static_cast<int>(h.H), h.hshift, w1, w2, kColsumRows,
            nb1, part1, part2);
        SAG_LAUNCH_CHECK();
    }
    gat_colsum_final<<<dim3(static_cast<unsigned>(cdiv(F, 64))), 256, 0, s>>>(part1, nb1, F, out1);
    SAG_LAUNCH_CHECK();
    gat_colsum_final<<<dim3(static_cast<unsigned>(cdiv(F, 64))), 256, 0, s>>>(part2, nb2, F, out2);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

// Saved forward state: Wh [n_ext, ldv(F)], el and er [n_ext, H], lse [n_local, H].
struct Saved {
    void* Wh = nullptr;
    float* el = nullptr;
    float* er = nullptr;
    float* lse = nullptr;
    size_t total = 0;
};

Saved carve_saved(void* base, int64_t n_local, int64_t n_ext, const Heads& h, sag_dtype dt) {
    Carver c(base, 0);
    Saved sv;
    sv.Wh = c.take<char>(dense_bytes(n_ext, h.F, dt));
    sv.el = c.take<float>(static_cast<size_t>(n_ext * h.H));
    sv.er = c.take<float>(static_cast<size_t>(n_ext * h.H));
    sv.lse = c.take<float>(static_cast<size_t>(n_local * h.H));
    sv.total = c.used();
    return sv;
}

struct FwdWs {
    void* Bp = nullptr;
    float* part = nullptr;
    size_t total = 0;
};

FwdWs carve_fwd(void* base, const sag_csr& A, int64_t d_in, const Heads& h, sag_dtype dt) {
    Carver c(base, 0);
    FwdWs w;
    w.Bp = c.take<char>(packed_b_bytes(d_in, 0, h.F, dt));
    w.part = c.take<float>(static_cast<size_t>(seg_count(A)) * partial_floats(h, dt));
    w.total = c.used();
    return w;
}

struct BwdWs {
    void* Bp = nullptr;
    void* gy = nullptr;
    float4* rinfo = nullptr;
    float* der = nullptr;
    void* dWh = nullptr;
    float* del = nullptr;
    float* part = nullptr;
    float* cpart = nullptr;
    float* cpart2 = nullptr;
    void* tn = nullptr;
    size_t tn_bytes = 0;
    size_t total = 0;
};

BwdWs carve_bwd(void* base, const sag_csr& A, const sag_csr& AT, int64_t d_in, const Heads& h, sag_dtype dt) {
    const int64_t n_l = A.n_rows, n_ext = A.n_cols;
    Carver c(base, 0);
    BwdWs w;
    w.Bp = c.take<char>(packed_b_bytes(h.F, 0, d_in, dt));
    w.gy = c.take<char>(dense_bytes(n_l, h.F, dt));
    w.rinfo = c.take<float4>(static_cast<size_t>(n_l * h.H));
    w.der = c.take<float>(static_cast<size_t>(n_l * h.H));
    w.dWh = c.take<char>(dense_bytes(n_ext, h.F, dt));
    w.del = c.take<float>(static_cast<size_t>(n_ext * h.H));
    const int64_t ns = std::max(seg_count(A), seg_count(AT));
    w.part = c.take<float>(static_cast<size_t>(ns) * partial_floats(h, dt));
    w.cpart = c.take<float>(static_cast<size_t>(std::max<int64_t>(colsum_blocks(n_ext), 1)) * h.F);
    w.cpart2 = c.take<float>(static_cast<size_t>(std::max<int64_t>(colsum_blocks(n_l), 1)) * h.F);
    w.tn_bytes = gemm_tn_ws_bytes(n_ext, ldv(d_in, dt), h.F, dt);
    w.tn = c.take<char>(w.tn_bytes);
    w.total = c.used();
    return w;
}

template <class T>
sag_status forward_typed(const sag_csr& A, const Heads& h, const Saved& sv, int64_t ldwh, const float* a_src,
                         const float* a_dst, const float* b, float slope, int relu, void* Out, int64_t ldo,
                         float* part, sag_dtype dt, hipStream_t s) {
    const int64_t n_l = A.n_rows, n_ext = A.n_cols;
    const int64_t es = elt_size(dt);
    SAG_TRY(launch_scores<T>(h, sv.Wh, ldwh, n_ext, a_src, a_dst, sv.el, sv.er, s));
    GatArgs p{};
    p.H = static_cast<int>(h.H);
    p.slope = slope;
    p.el = sv.el;
    p.er = sv.er;
    p.a_src = a_src;
    p.part = part;
    p.ldp = partial_floats(h, dt);
    p.C = h.C;
    p.hshift = h.hshift;
    p.soff = h.C * static_cast<int>(vec_elems(dt));
    p.X = sv.Wh;
    p.ldx = ldwh;
    p.o_lse = sv.lse;
    p.y = Out;
    p.ldy = ldo;
    p.bias = b;
    p.relu = relu;
    const int64_t bytes = 8 * (n_l + 1) + 4 * A.nnz + es * h.F * (n_ext + n_l) + 4 * h.H * 2 * n_l;
    TraceScope trace(trace_enabled() ? shape_name("gat_fwd", dt == SAG_BF16 ? "bf16" : "f32", n_l, A.nnz, h.F)
                                     : std::string(),
                     s, bytes, 2 * A.nnz * h.F);
    return launch_pass<M_FWD, T>(A, p, s);
}

template <class T>
sag_status backward_typed(const sag_csr& A, const sag_csr& AT, const Heads& h, const Saved& sv, int64_t ldwh,
                          const float* a_src, const float* a_dst, float slope, int relu, const void* Y,
                          const void* G_out, int64_t ldg, float* da_src, float* da_dst, float* db,
                          const BwdWs& w, sag_dtype dt, hipStream_t s) {
    const int64_t n_l = A.n_rows, n_ext = A.n_cols;
    const int64_t es = elt_size(dt);
    const int64_t ldf = ldv(h.F, dt);
    const void* GY = relu ? w.gy : G_out;
    const int64_t ldgy = relu ? ldf : ldg;
    GatArgs p{};
    p.C = h.C;
    p.H = static_cast<int>(h.H);
    p.hshift = h.hshift;
    p.slope = slope;
    p.el = sv.el;
    p.er = sv.er;
    p.lse = sv.lse;
    p.a_src = a_src;
    p.part = w.part;
    p.ldp = partial_floats(h, dt);
    p.soff = h.C * static_cast<int>(vec_elems(dt));
    p.n_local = n_l;
    {
        GatArgs q = p;
        q.X = sv.Wh;
        q.ldx = ldwh;
        q.own = G_out;
        q.ldown = ldg;
        q.ymask = relu ? Y : nullptr;
        q.ldym = ldg;
        q.gy = relu ? w.gy : nullptr;
        q.ldgy = ldf;
        q.o_rinfo = w.rinfo;
        q.o_der = w.der;
        const int64_t bytes = 8 * (n_l + 1) + 4 * A.nnz + es * h.F * (n_ext + n_l * (relu ? 3 : 1)) +
                              4 * h.H * 2 * n_l + 20 * h.H * n_l;
        TraceScope trace(trace_enabled() ? shape_name("gat_bwd_rows", dt == SAG_BF16 ? "bf16" : "f32", n_l, A.nnz, h.F)
                                         : std::string(),
                         s, bytes, 2 * A.nnz * h.F);
        SAG_TRY((launch_pass<M_BWA, T>(A, q, s)));
    }
    {
        GatArgs q = p;
        q.X = GY;
        q.ldx = ldgy;
        q.own = sv.Wh;
        q.ldown = ldwh;
        q.rinfo = w.rinfo;
        q.der = w.der;
        q.o_del = w.del;
        q.y = w.dWh;
        q.ldy = ldf;
        q.a_src = a_src;
        q.a_dst = a_dst;
        const int64_t bytes = 8 * (n_ext + 1) + 4 * AT.nnz + es * h.F * (n_l + 2 * n_ext) + 20 * h.H * n_l +
                              8 * h.H * n_ext;
        TraceScope trace(trace_enabled() ? shape_name("gat_bwd_cols", dt == SAG_BF16 ? "bf16" : "f32", n_ext, AT.nnz,
                                                      h.F)
                                         : std::string(),
                         s, bytes, 4 * AT.nnz * h.F);
        SAG_TRY((launch_pass<M_BWT, T>(AT, q, s)));
    }
    TraceScope trace(trace_enabled() ? shape_name("gat_colsums", dt == SAG_BF16 ? "bf16" : "f32", n_ext, h.F, 0)
                                     : std::string(),
                     s, es * h.F * (2 * n_l + n_ext) + 4 * h.H * (n_l + n_ext), 0);
    if (db) SAG_TRY(launch_colsum<T>(h, GY, ldgy, n_l, nullptr, w.cpart, db, s));
    if (da_dst && da_src) {
        SAG_TRY(launch_colsum2<T>(h, sv.Wh, ldwh, n_l, w.der, w.cpart2, da_dst, n_ext, w.del, w.cpart, da_src, s));
    } else {
        if (da_dst) SAG_TRY(launch_colsum<T>(h, sv.Wh, ldwh, n_l, w.der, w.cpart, da_dst, s));
        if (da_src) SAG_TRY(launch_colsum<T>(h, sv.Wh, ldwh, n_ext, w.del, w.cpart, da_src, s));
    }
    return SAG_OK;
}

}  // namespace
}  // namespace sag

using namespace sag;

extern "C" size_t sag_gat_save_bytes(int64_t n_local, int64_t n_ext, int64_t heads, int64_t d_head, sag_dtype dt) {
    Heads h;
    if (n_local < 0 || n_ext < n_local || heads_of("gat", heads, d_head, dt, &h) != SAG_OK) return 0;
    return carve_saved(nullptr, n_local, n_ext, h, dt).total;
}

extern "C" size_t sag_gat_forward_workspace_bytes(const sag_csr* A, int64_t d_in, int64_t heads, int64_t d_head,
                                                  sag_dtype dt) {
    Heads h;
    if (!A || d_in <= 0 || heads_of("gat", heads, d_head, dt, &h) != SAG_OK) return 0;
    return carve_fwd(nullptr, *A, d_in, h, dt).total;
}

extern "C" sag_status sag_gat_layer_forward(const sag_csr* A, const void* H_ext, int64_t ldh, int64_t d_in,
                                            const void* W, const float* a_src, const float* a_dst, const float* b,
                                            int64_t heads, int64_t d_head, float slope, int relu, sag_dtype dt,
                                            void* Out, int64_t ldo, void* save, size_t save_bytes, void* ws,
                                            size_t ws_bytes, void* stream) {
    Heads h;
    SAG_TRY(heads_of("gat_forward", heads, d_head, dt, &h));
    SAG_TRY(check_csr("gat_forward", A));
    if (d_in <= 0) return fail(SAG_E_INVALID, "gat_forward: d_in must be positive");
    if (!nn_k_fits(d_in, 0, dt)) return fail(SAG_E_UNSUPPORTED, "gat_forward: d_in too large for the transform");
    if (A->n_cols < A->n_rows) return fail(SAG_E_INVALID, "gat_forward: fewer columns than local rows");
    if (!W || !a_src || !a_dst) return fail(SAG_E_INVALID, "gat_forward: null W or attention vector");
    if (!std::isfinite(slope)) return fail(SAG_E_INVALID, "gat_forward: slope must be finite");
    const int64_t n_l = A->n_rows, n_ext = A->n_cols;
    SAG_TRY(check_dense("gat_forward H_ext", H_ext, n_ext, d_in, ldh, dt));
    SAG_TRY(check_dense("gat_forward Out", Out, n_l, h.F, ldo, dt));
    const Saved need_sv = carve_saved(nullptr, n_l, n_ext, h, dt);
    if (save_bytes < need_sv.total || !save) return fail(SAG_E_WORKSPACE, "gat_forward: save buffer too small");
    if (!aligned16(save)) return fail(SAG_E_ALIGN, "gat_forward: save not 16-B aligned");
    const FwdWs need = carve_fwd(nullptr, *A, d_in, h, dt);
    if (ws_bytes < need.total || !ws) return fail(SAG_E_WORKSPACE, "gat_forward: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "gat_forward: workspace not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Saved sv = carve_saved(save, n_l, n_ext, h, dt);
    const FwdWs w = carve_fwd(ws, *A, d_in, h, dt);
    const int64_t ldwh = ldv(h.F, dt);

    // Wh = H_ext W
    PackSrc src;
    src.p[0][0] = W;
    src.sk[0][0] = h.F;
    src.sn[0][0] = 1;
    NLayout nl;
    nl.n0 = nl.nsplit = h.F;
    SAG_TRY(pack_b(src, d_in, 0, nl, dt, w.Bp, s));
    GemmA a;
    a.a1 = H_ext; a.lda1 = ldh; a.k1 = d_in; a.m1 = n_ext;
    SAG_TRY(gemm_run(n_ext, h.F, a, w.Bp, dt, sv.Wh, ldwh, Epilogue{}, s));
    if (dt == SAG_BF16)
        return forward_typed<uint16_t>(*A, h, sv, ldwh, a_src, a_dst, b, slope, relu, Out, ldo, w.part, dt, s);
    return forward_typed<float>(*A, h, sv, ldwh, a_src, a_dst, b, slope, relu, Out, ldo, w.part, dt, s);
}

extern "C" size_t sag_gat_backward_workspace_bytes(const sag_csr* A, const sag_csr* AT, int64_t d_in, int64_t heads,
                                                   int64_t d_head, sag_dtype dt) {
    Heads h;
    if (!A || !AT || d_in <= 0 || heads_of("gat", heads, d_head, dt, &h) != SAG_OK) return 0;
    return carve_bwd(nullptr, *A, *AT, d_in, h, dt).total;
}

extern "C" sag_status sag_gat_layer_backward(const sag_csr* A, const sag_csr* AT, const void* H_ext, int64_t ldh,
                                             int64_t d_in, const void* W, const float* a_src, const float* a_dst,
                                             int64_t heads, int64_t d_head, float slope, int relu, const void* Y,
                                             const void* G_out, int64_t ldg, float* dW, float* da_src,
                                             float* da_dst, float* db, void* dH_ext, int64_t ldd, sag_dtype dt,
                                             const void* save, size_t save_bytes, void* ws, size_t ws_bytes,
                                             void* stream) {
    Heads h;
    SAG_TRY(heads_of("gat_backward", heads, d_head, dt, &h));
    SAG_TRY(check_csr("gat_backward", A));
    SAG_TRY(check_csr("gat_backward", AT));
    if (d_in <= 0) return fail(SAG_E_INVALID, "gat_backward: d_in must be positive");
    const int64_t n_l = A->n_rows, n_ext = A->n_cols;
    if (n_ext < n_l) return fail(SAG_E_INVALID, "gat_backward: fewer columns than local rows");
    if (AT->n_rows != n_ext || AT->n_cols != n_l || AT->nnz != A->nnz)
        return fail(SAG_E_INVALID, "gat_backward: AT is not the transpose's shape of A");
    if (!W || !a_src || !a_dst) return fail(SAG_E_INVALID, "gat_backward: null W or attention vector");
    if (!std::isfinite(slope)) return fail(SAG_E_INVALID, "gat_backward: slope must be finite");
    if (dH_ext && !nn_k_fits(h.F, 0, dt))
        return fail(SAG_E_UNSUPPORTED, "gat_backward: heads * d_head too large for the input-gradient product");
    if (dW) SAG_TRY(check_dense("gat_backward H_ext", H_ext, n_ext, d_in, ldh, dt));
    SAG_TRY(check_dense("gat_backward G_out", G_out, n_l, h.F, ldg, dt));
    if (relu) SAG_TRY(check_dense("gat_backward Y", Y, n_l, h.F, ldg, dt));
    if (dH_ext) SAG_TRY(check_dense("gat_backward dH_ext", dH_ext, n_ext, d_in, ldd, dt));
    const Saved need_sv = carve_saved(nullptr, n_l, n_ext, h, dt);
    if (save_bytes < need_sv.total || !save) return fail(SAG_E_INVALID, "gat_backward: missing saved forward state");
    if (!aligned16(save)) return fail(SAG_E_ALIGN, "gat_backward: save not 16-B aligned");
    const BwdWs need = carve_bwd(nullptr, *A, *AT, d_in, h, dt);
    if (ws_bytes < need.total || !ws) return fail(SAG_E_WORKSPACE, "gat_backward: workspace too small");
    if (!aligned16(ws)) return fail(SAG_E_ALIGN, "gat_backward: workspace not 16-B aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const Saved sv = carve_saved(const_cast<void*>(save), n_l, n_ext, h, dt);
    const BwdWs w = carve_bwd(ws, *A, *AT, d_in, h, dt);
    const int64_t ldwh = ldv(h.F, dt), ldf = ldv(h.F, dt);
    if (dt == SAG_BF16)
        SAG_TRY(backward_typed<uint16_t>(*A, *AT, h, sv, ldwh, a_src, a_dst, slope, relu, Y, G_out, ldg, da_src,
                                         da_dst, db, w, dt, s));
    else
        SAG_TRY(backward_typed<float>(*A, *AT, h, sv, ldwh, a_src, a_dst, slope, relu, Y, G_out, ldg, da_src, da_dst,
                                      db, w, dt, s));
    if (dW) {
        GemmA x;
        x.a1 = H_ext; x.lda1 = ldh; x.k1 = d_in; x.m1 = n_ext;
        SAG_TRY(gemm_tn_run(n_ext, h.F, x, w.dWh, ldf, nullptr, 0, dW, h.F, nullptr, dt, w.tn, w.tn_bytes, s));
    }
    if (!dH_ext) return SAG_OK;
    // dH_ext = dWh W^T: element (k, n) of the packed operand is W[n, k]
    PackSrc src;
    src.p[0][0] = W;
    src.sk[0][0] = 1;
    src.sn[0][0] = h.F;
    NLayout nl;
    nl.n0 = nl.nsplit = d_in;
    SAG_TRY(pack_b(src, h.F, 0, nl, dt, w.Bp, s));
    GemmA g;
    g.a1 = w.dWh; g.lda1 = ldf; g.k1 = h.F; g.m1 = n_ext;
    return gemm_run(n_ext, d_in, g, w.Bp, dt, dH_ext, ldd, Epilogue{}, s);
}
