// Row-gather probe: the rate at which the memory system delivers the rows an
// SpMM gathers, measured without the SpMM's row structure, values or epilogue.
//
// Every wavefront takes an equal, contiguous chunk of the id list and reads
// the rows those ids name, in order, with the SpMM's lane layout (one group
// of G lanes per row, one 16-byte vector per lane and step, eight rows in
// flight per group), so the two kernels issue the same loads for the same
// access pattern.  The data read is folded into a per-lane sum that goes to a
// small sink, which keeps the loads live and gives a test a defined result.
#include "common.h"

namespace sag {

// Compute units of the current device (api.cpp), queried once per process.
int device_cus();

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 4;

int probe_waves() { return device_cus() * kProbeBlocksPerCu * (kProbeThreads / 64); }

__device__ __forceinline__ void add_vec(uint4& a, const uint4& x, bool ok) {
    a.x += ok ? x.x : 0u;
    a.y += ok ? x.y : 0u;
    a.z += ok ? x.z : 0u;
    a.w += ok ? x.w : 0u;
}

// G lanes per row, NV 16-B vectors per lane and row (C = vectors per row).
template <int G, int NV>
__global__ __launch_bounds__(kProbeThreads) void gather_probe(const uint4* __restrict__ X, int64_t ld16, int C,
                                                              const int32_t* __restrict__ ids, int64_t n,
                                                              int64_t chunk, uint4* __restrict__ sink) {
    constexpr int P = 64 / G;
    constexpr int U = 8 / NV;
    const int lane = threadIdx.x & 63;
    const int gl = lane % G, grp = lane / G;
    const int64_t wave = (static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x) >> 6;
    const int64_t beg = wave * chunk;
    const int64_t end = beg + chunk < n ? beg + chunk : n;
    int ch[NV];
    bool vok[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        vok[v] = v * G + gl < C;
        ch[v] = vok[v] ? v * G + gl : C - 1;
    }
    uint4 acc = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t i0 = beg; i0 < end; i0 += 64) {
        const int m = static_cast<int>(end - i0 < 64 ? end - i0 : 64);
        const int32_t my = ids[i0 + (lane < m ? lane : m - 1)];
        for (int t = 0; t < m; t += P * U) {
            uint4 x[U][NV];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = t + u * P + grp;
                ok[u] = e < m;
                const int32_t c = __shfl(my, e < m ? e : m - 1, 64);
#pragma unroll
                for (int v = 0; v < NV; ++v) x[u][v] = X[static_cast<int64_t>(c) * ld16 + ch[v]];
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < NV; ++v) add_vec(acc, x[u][v], ok[u] && vok[v]);
        }
    }
    sink[wave * 64 + lane] = acc;
}

template <int G, int NV>
sag_status launch_probe(const uint4* X, int64_t ld16, int C, const int32_t* ids, int64_t n, int64_t chunk,
                        uint4* sink, hipStream_t s) {
    gather_probe<G, NV><<<dim3(static_cast<unsigned>(device_cus() * kProbeBlocksPerCu)), kProbeThreads, 0, s>>>(
        X, ld16, C, ids, n, chunk, sink);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace
}  // namespace sag

using namespace sag;

extern "C" size_t sag_gather_probe_sink_bytes(void) {
    return static_cast<size_t>(probe_waves()) * 64 * sizeof(uint4);
}

extern "C" sag_status sag_gather_probe(const void* X, int64_t ldx, int64_t d, sag_dtype dt, const int32_t* ids,
                                       int64_t n, void* sink, size_t sink_bytes, void* stream) {
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "gather_probe: bad dtype");
    if (n < 0 || d < 1) return fail(SAG_E_INVALID, "gather_probe: bad sizes");
    if (n > 0 && (!X || !ids)) return fail(SAG_E_INVALID, "gather_probe: null pointer");
    if (!sink || sink_bytes < sag_gather_probe_sink_bytes()) return fail(SAG_E_WORKSPACE, "gather_probe: sink too small");
    if (!aligned16(sink)) return fail(SAG_E_ALIGN, "gather_probe: sink not 16-B aligned");
    const int64_t es = elt_size(dt);
    if (n > 0 && (!aligned16(X) || (ldx * es) % 16 != 0)) return fail(SAG_E_ALIGN, "gather_probe: X or its pitch not 16-B aligned");
    if (ldx < d) return fail(SAG_E_INVALID, "gather_probe: ldx < d");
    const int64_t C = cdiv(d * es, 16);
    if (C > 256) return fail(SAG_E_UNSUPPORTED, "gather_probe: rows wider than 4 KB");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t W = probe_waves();
    const int64_t chunk = round_up(cdiv(n > 0 ? n : 1, W), 64);
    const uint4* Xv = static_cast<const uint4*>(X);
    const int64_t ld16 = ldx * es / 16;
    uint4* sk = static_cast<uint4*>(sink);
    const int c = static_cast<int>(C);
    if (C <= 1) return launch_probe<1, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 2) return launch_probe<2, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 4) return launch_probe<4, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 8) return launch_probe<8, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 16) return launch_probe<16, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 32) return launch_probe<32, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 64) return launch_probe<64, 1>(Xv, ld16, c, ids, n, chunk, sk, s);
    if (C <= 128) return launch_probe<64, 2>(Xv, ld16, c, ids, n, chunk, sk, s);
    return launch_probe<64, 4>(Xv, ld16, c, ids, n, chunk, sk, s);
}
