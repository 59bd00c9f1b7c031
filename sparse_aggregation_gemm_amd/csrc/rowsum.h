// Row sums of a CSR times a dense matrix, shared by the SpMM and the fused
// aggregate -> transform kernel: 16-byte feature loads, a group of G lanes
// per row of X (G the power of two >= the row's vector count C, at most 64;
// wider rows give each lane NV vectors), column indices and values loaded
// one per lane and handed out with lane shuffles so that each lane keeps
// several independent loads in flight, fp32 accumulation in a fixed order.
#pragma once

#include "common.h"

namespace sag {
namespace rowsum {

template <class XT>
__device__ __forceinline__ uint4 load_x(const XT* X, int64_t ldx, int32_t c, int ch) {
    return *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(c) * ldx + ch * Vec<XT>::N);
}

template <class XT, int NV, int U>
__device__ __forceinline__ void accumulate(const XT* X, int64_t ldx, const int (&ch)[NV],
                                           const int32_t (&c)[U], const float (&w)[U],
                                           const bool (&ok)[U], float (&acc)[NV][Vec<XT>::N]) {
    constexpr int V = Vec<XT>::N;
    uint4 x[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) x[u][v] = load_x(X, ldx, c[u], ch[v]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            float f[V];
            unpack<XT>(x[u][v], f);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float t = fmaf(w[u], f[k], acc[v][k]);
                acc[v][k] = ok[u] ? t : acc[v][k];
            }
        }
    }
}

__device__ __forceinline__ int64_t rec_start(const int4& r) {
    return static_cast<int64_t>(static_cast<uint64_t>(static_cast<uint32_t>(r.z)) |
                                (static_cast<uint64_t>(static_cast<uint32_t>(r.w)) << 32));
}

// Sums entries [start, start + len) of one row across the whole wavefront:
// group g takes entries g, g + P, ...; every lane ends with the full sum of its vectors.
template <class XT, int G, int NV>
__device__ __forceinline__ void wave_row_sum(const XT* X, int64_t ldx, int C,
                                             const int32_t* idx, const float* val, int64_t start, int len,
                                             float (&acc)[NV][Vec<XT>::N]) {
    constexpr int V = Vec<XT>::N;
    constexpr int P = 64 / G;
    constexpr int U = NV >= 4 ? 2 : (NV >= 2 ? 4 : 8);
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    int ch[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) ch[v] = min(v * G + gl, C - 1);
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int k = 0; k < V; ++k) acc[v][k] = 0.f;
    for (int j0 = 0; j0 < len; j0 += 64) {
        const int jj = j0 + lane;
        const bool mine = jj < len;
        const int32_t c_my = mine ? idx[start + jj] : 0;
        const float v_my = mine ? (val ? val[start + jj] : 1.f) : 0.f;
        const int nh = min(64, len - j0);
        for (int t = 0; t < nh; t += U * P) {
            int32_t c[U];
            float w[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int src = t + u * P + grp;
                const int s2 = min(src, 63);
                c[u] = __shfl(c_my, s2, 64);
                w[u] = __shfl(v_my, s2, 64);
                ok[u] = src < nh;
            }
            accumulate<XT, NV, U>(X, ldx, ch, c, w, ok, acc);
        }
    }
    // add the P group sums with a fixed butterfly
#pragma unroll
    for (int off = G; off < 64; off <<= 1)
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
            for (int k = 0; k < V; ++k) acc[v][k] += __shfl_xor(acc[v][k], off, 64);
}

// Sums entries [start, start + len) of one row for a group of G lanes (P =
// 64 / G rows per wavefront, one per group; lmax is the wavefront's longest
// len, so every lane runs the same loop).
template <class XT, int G, int NV>
__device__ __forceinline__ void group_row_sum(const XT* X, int64_t ldx, int C, const int32_t* idx,
                                              const float* val, int64_t start, int len, int lmax,
                                              float (&acc)[NV][Vec<XT>::N]) {
    constexpr int V = Vec<XT>::N;
    constexpr int U = NV >= 4 ? 2 : (NV >= 2 ? 4 : 8);
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    int ch[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) ch[v] = min(v * G + gl, C - 1);
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int k = 0; k < V; ++k) acc[v][k] = 0.f;
    for (int j0 = 0; j0 < lmax; j0 += G) {
        const int jj = j0 + gl;
        const bool mine = jj < len;
        const int32_t c_my = mine ? idx[start + jj] : 0;
        const float v_my = mine ? (val ? val[start + jj] : 1.f) : 0.f;
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
            accumulate<XT, NV, U>(X, ldx, ch, c, w, ok, acc);
        }
    }
}

}  // namespace rowsum
}  // namespace sag
