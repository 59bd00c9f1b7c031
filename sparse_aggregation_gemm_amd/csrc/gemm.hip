// Dense products of a GNN layer on the matrix cores (CAGNET page: after the
// SpMM, each process multiplies its rows by the weight matrix; the backward
// pass uses the same primitives for the weight and input gradients).
//
//   gemm_nn : C[M, N] = [A1 | A2] B  + epilogue (bias, addend, ReLU)
//             -- the forward transform and the input-gradient product.
//   gemm_tn : C[K, N] = [A1 | A2]^T B -- the weight gradient; the reduction
//             runs over the M rows, split into chunks whose fp32 partials are
//             added in chunk order by a second kernel (deterministic).
//
// bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2f32; both
// accumulate in fp32.  Tiles are staged through LDS; the next k-tile is
// loaded into registers while the current one feeds the MFMAs.  B (the
// weight, tiny next to A) is first packed into a zero-padded [N_pad, K_pad]
// k-contiguous array, so the main loops need no bounds checks on it.
// Workgroups are renumbered so that the tiles sharing rows of A run on the
// same XCD (one L2 each on MI355X).
#include "ops.h"
#include "trace.h"

namespace sag {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kKPad = 32;    // K of a packed B is padded to this
constexpr int kNPad = 256;   // N of a packed B is padded to this

inline int64_t kp(int64_t k, sag_dtype dt) { return round_up(k, vec_elems(dt)); }
inline int64_t k_total(int64_t k1, int64_t k2, sag_dtype dt) { return round_up(kp(k1, dt) + kp(k2, dt), kKPad); }

// ---- element tricks on 16-byte vectors ---------------------------------------------

// Zeroes elements >= n of a vector of T.
template <class T>
__device__ __forceinline__ uint4 keep_first(uint4 v, int n) {
    constexpr int V = Vec<T>::N;
    if (n >= V) return v;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (V == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (e >= n) w[e] = 0;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (e >= n) w[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Zeroes the elements of a whose mask element is not > 0 (NaN counts as not).
template <class T>
__device__ __forceinline__ uint4 apply_mask(uint4 a, uint4 m) {
    uint32_t aw[4] = {a.x, a.y, a.z, a.w};
    const uint32_t mw[4] = {m.x, m.y, m.z, m.w};
    if constexpr (Vec<T>::N == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t b = mw[e];
            if (!(b >= 1u && b <= 0x7f800000u)) aw[e] = 0;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b = (e & 1) ? (mw[e / 2] >> 16) : (mw[e / 2] & 0xffffu);
            if (!(b >= 1u && b <= 0x7f80u)) aw[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
    }
    return make_uint4(aw[0], aw[1], aw[2], aw[3]);
}

// Loads the 16-byte vector of virtual column k0 (a multiple of V) of row r
// of the block operand [A1 | A2]; zero outside the operand.
template <class T>
struct AOperand {
    const T* a1;
    int64_t lda1, k1, m1, k1p;
    const T* a2;
    int64_t lda2, k2, k2p;
    const T* mask;
    int64_t ldmask;
    int64_t M;

    __device__ __forceinline__ uint4 load(int64_t r, int64_t k0) const {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r >= M) return v;
        if (k0 < k1p) {
            if (r < m1) {
                v = *reinterpret_cast<const uint4*>(a1 + r * lda1 + k0);
                v = keep_first<T>(v, static_cast<int>(k1 - k0));
                if (mask) v = apply_mask<T>(v, *reinterpret_cast<const uint4*>(mask + r * ldmask + k0));
            }
        } else if (k0 < k1p + k2p) {
            const int64_t kk = k0 - k1p;
            v = *reinterpret_cast<const uint4*>(a2 + r * lda2 + kk);
            v = keep_first<T>(v, static_cast<int>(k2 - kk));
        }
        return v;
    }
};

template <class T>
AOperand<T> make_aop(const GemmA& A, int64_t M, sag_dtype dt) {
    AOperand<T> o;
    o.a1 = static_cast<const T*>(A.a1);
    o.lda1 = A.lda1;
    o.k1 = A.k1;
    o.m1 = A.a1 ? (A.m1 > 0 ? A.m1 : M) : 0;
    o.k1p = kp(A.k1, dt);
    o.a2 = static_cast<const T*>(A.a2);
    o.lda2 = A.lda2;
    o.k2 = A.a2 ? A.k2 : 0;
    o.k2p = A.a2 ? kp(A.k2, dt) : 0;
    o.mask = static_cast<const T*>(A.mask);
    o.ldmask = A.ldmask;
    o.M = M;
    return o;
}

// MFMA traits: k per instruction and fragment loads from LDS rows with k
// contiguous.
template <class T> struct Mfma;
template <> struct Mfma<uint16_t> {
    static constexpr int KI = 16;   // k per instruction
    using frag = bf16x8_t;
    __device__ static __forceinline__ frag ld(const uint16_t* row, int k) {
        return *reinterpret_cast<const bf16x8_t*>(row + k + (threadIdx.x & 63) / 32 * 8);
    }
    __device__ static __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KI = 2;
    using frag = float;
    __device__ static __forceinline__ frag ld(const float* row, int k) {
        return row[k + (threadIdx.x & 63) / 32];
    }
    __device__ static __forceinline__ f32x16_t mma(frag a, frag b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// Workgroup id -> logical tile id with the tiles of one XCD contiguous
// (workgroups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t total) {
    constexpr int64_t X = 8;
    const int64_t per = total / X, rem = total % X;
    const int64_t xcd = bid % X, local = bid / X;
    return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}

template <class T>
struct EpiT {
    T* c;
    int64_t ldc;
    T* pre;
    const T* add;
    int64_t ld_add, n_add;
    const float* bias;
    int relu;
};

// ---- NN ------------------------------------------------------------------------------
constexpr int kBM = 128;

template <class T, int BN>
__global__ __launch_bounds__(256) void gemm_nn(AOperand<T> A, const T* __restrict__ Bp, int64_t Kt,
                                               int64_t N, int64_t n_nblk, EpiT<T> e) {
    constexpr int V = Vec<T>::N;
    constexpr int BK = 64 / sizeof(T);          // 64 bytes of k per row and tile
    constexpr int LP = BK + V;                  // LDS row pitch (elements), +16 B
    constexpr int NB = BN / 64;                 // 32-column blocks per wave
    constexpr int KI = Mfma<T>::KI;
    __shared__ __attribute__((aligned(16))) T As[kBM * LP];
    __shared__ __attribute__((aligned(16))) T Bs[BN * LP];

    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t mb0 = (tile / n_nblk) * kBM;
    const int64_t nb0 = (tile % n_nblk) * BN;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wm = wave & 1, wn = wave >> 1;

    uint4 ra[2], rb[NB];
    auto load_tile = [&](int64_t kt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = t + 256 * i;
            ra[i] = A.load(mb0 + q / 4, kt * BK + (q % 4) * V);
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int q = t + 256 * i;
            rb[i] = *reinterpret_cast<const uint4*>(Bp + (nb0 + q / 4) * Kt + kt * BK + (q % 4) * V);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int q = t + 256 * i;
            *reinterpret_cast<uint4*>(&As[(q / 4) * LP + (q % 4) * V]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int q = t + 256 * i;
            *reinterpret_cast<uint4*>(&Bs[(q / 4) * LP + (q % 4) * V]) = rb[i];
        }
    };

    f32x16_t acc[2][NB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int64_t nkt = Kt / BK;
    load_tile(0);
    store_tile();
    __syncthreads();
    for (int64_t kt = 0; kt < nkt; ++kt) {
        if (kt + 1 < nkt) load_tile(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK; ks += KI) {
            typename Mfma<T>::frag fa[2], fb[NB];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = Mfma<T>::ld(&As[(wm * 64 + i * 32 + lane % 32) * LP], ks);
#pragma unroll
            for (int j = 0; j < NB; ++j) fb[j] = Mfma<T>::ld(&Bs[(wn * (BN / 2) + j * 32 + lane % 32) * LP], ks);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NB; ++j) acc[i][j] = Mfma<T>::mma(fa[i], fb[j], acc[i][j]);
        }
        __syncthreads();
        if (kt + 1 < nkt) {
            store_tile();
            __syncthreads();
        }
    }

    // epilogue: acc register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
    // column l%32 of its 32x32 block
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t col = nb0 + wn * (BN / 2) + j * 32 + lane % 32;
            if (col >= N) continue;
            const float bias = e.bias ? e.bias[col] : 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = mb0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                if (row >= A.M) continue;
                float y = acc[i][j][r] + bias;
                if (e.add && row < e.n_add) y += to_f32(e.add[row * e.ld_add + col]);
                if (e.pre) e.pre[row * e.ldc + col] = from_f32<T>(y);
                if (e.relu) y = y < 0.f ? 0.f : y;
                e.c[row * e.ldc + col] = from_f32<T>(y);
            }
        }
    }
}

// ---- TN (weight gradient) -----------------------------------------------------------
// Tile: BKT rows of C (the K dimension) x BNT columns, reduction over a
// chunk of M rows, MS rows per step.
constexpr int kBKT = 128;

template <class T, int BNT>
__global__ __launch_bounds__(256) void gemm_tn(AOperand<T> A, const T* __restrict__ B, int64_t ldb,
                                               const T* __restrict__ mask, int64_t ldmask, int64_t N,
                                               int64_t n_ktile, int64_t n_ntile, int64_t rows_per_chunk,
                                               float* __restrict__ part, int64_t ldp_k, int64_t ldp_n,
                                               float* __restrict__ part_cs) {
    constexpr int V = Vec<T>::N;
    constexpr int KI = Mfma<T>::KI;
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int MS = kBf16 ? 32 : 16;               // M rows per step
    constexpr int NBK = kBKT / 64, NBN = BNT / 64;    // 32-blocks per wave
    // bf16: LDS transposed [k][m] and [n][m]; fp32: natural [m][k] and [m][n]
    constexpr int LPA = kBf16 ? MS + 8 : kBKT + 4;
    constexpr int LPB = kBf16 ? MS + 8 : BNT + 4;
    constexpr int SA = kBf16 ? kBKT * LPA : MS * LPA;
    constexpr int SB = kBf16 ? BNT * LPB : MS * LPB;
    __shared__ __attribute__((aligned(16))) T As[SA];
    __shared__ __attribute__((aligned(16))) T Bs[SB];
    constexpr int VA = MS * kBKT / V / 256;           // A vectors per thread per step
    constexpr int VB = MS * BNT / V / 256;
    static_assert(VA >= 1 && VB >= 1, "tile too small");

    const int64_t tiles = n_ktile * n_ntile;
    const int64_t chunk = blockIdx.x / tiles;
    const int64_t tt = blockIdx.x % tiles;
    const int64_t k0 = (tt / n_ntile) * kBKT;
    const int64_t n0 = (tt % n_ntile) * BNT;
    const int64_t m_begin = chunk * rows_per_chunk;
    const int64_t m_end = min(A.M, m_begin + rows_per_chunk);
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wk = wave & 1, wn = wave >> 1;
    const bool do_cs = part_cs && k0 == 0;

    uint4 ra[VA], rb[VB];
    auto load_step = [&](int64_t m0) {
#pragma unroll
        for (int i = 0; i < VA; ++i) {
            const int q = t + 256 * i;
            const int r = q / (kBKT / V), c = (q % (kBKT / V)) * V;
            ra[i] = (m0 + r < m_end) ? A.load(m0 + r, k0 + c) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = t + 256 * i;
            const int r = q / (BNT / V), c = (q % (BNT / V)) * V;
            const int64_t row = m0 + r, col = n0 + c;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row < m_end && col < N) {
                v = *reinterpret_cast<const uint4*>(B + row * ldb + col);
                v = keep_first<T>(v, static_cast<int>(N - col));
                if (mask) v = apply_mask<T>(v, *reinterpret_cast<const uint4*>(mask + row * ldmask + col));
            }
            rb[i] = v;
        }
    };
    auto store_step = [&]() {
#pragma unroll
        for (int i = 0; i < VA; ++i) {
            const int q = t + 256 * i;
            const int r = q / (kBKT / V), c = (q % (kBKT / V)) * V;
            if constexpr (kBf16) {
                const uint32_t w[4] = {ra[i].x, ra[i].y, ra[i].z, ra[i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    As[(c + e) * LPA + r] = static_cast<uint16_t>((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
            } else {
                *reinterpret_cast<uint4*>(&As[r * LPA + c]) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < VB; ++i) {
            const int q = t + 256 * i;
            const int r = q / (BNT / V), c = (q % (BNT / V)) * V;
            if constexpr (kBf16) {
                const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    Bs[(c + e) * LPB + r] = static_cast<uint16_t>((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
            } else {
                *reinterpret_cast<uint4*>(&Bs[r * LPB + c]) = rb[i];
            }
        }
    };

    f32x16_t acc[NBK][NBN];
#pragma unroll
    for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    float cs = 0.f;

    if (m_begin < m_end) {
        load_step(m_begin);
        store_step();
        __syncthreads();
        for (int64_t m0 = m_begin; m0 < m_end; m0 += MS) {
            const bool more = m0 + MS < m_end;
            if (more) load_step(m0 + MS);
            if (do_cs && t < BNT) {
                if constexpr (kBf16) {
                    for (int r = 0; r < MS; ++r) cs += bf16_to_f32(Bs[t * LPB + r]);
                } else {
                    for (int r = 0; r < MS; ++r) cs += Bs[r * LPB + t];
                }
            }
#pragma unroll
            for (int ks = 0; ks < MS; ks += KI) {
                typename Mfma<T>::frag fa[NBK], fb[NBN];
                if constexpr (kBf16) {
#pragma unroll
                    for (int i = 0; i < NBK; ++i)
                        fa[i] = Mfma<T>::ld(&As[(wk * (kBKT / 2) + i * 32 + lane % 32) * LPA], ks);
#pragma unroll
                    for (int j = 0; j < NBN; ++j)
                        fb[j] = Mfma<T>::ld(&Bs[(wn * (BNT / 2) + j * 32 + lane % 32) * LPB], ks);
                } else {
                    const int mr = ks + lane / 32;
#pragma unroll
                    for (int i = 0; i < NBK; ++i)
                        fa[i] = reinterpret_cast<const float*>(As)[mr * LPA + wk * (kBKT / 2) + i * 32 + lane % 32];
#pragma unroll
                    for (int j = 0; j < NBN; ++j)
                        fb[j] = reinterpret_cast<const float*>(Bs)[mr * LPB + wn * (BNT / 2) + j * 32 + lane % 32];
                }
#pragma unroll
                for (int i = 0; i < NBK; ++i)
#pragma unroll
                    for (int j = 0; j < NBN; ++j) acc[i][j] = Mfma<T>::mma(fa[i], fb[j], acc[i][j]);
            }
            __syncthreads();
            if (more) {
                store_step();
                __syncthreads();
            }
        }
    }

    float* out = part + chunk * ldp_k * ldp_n;
#pragma unroll
    for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j) {
            const int64_t col = n0 + wn * (BNT / 2) + j * 32 + lane % 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = k0 + wk * (kBKT / 2) + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                out[row * ldp_n + col] = acc[i][j][r];
            }
        }
    if (do_cs && t < BNT) part_cs[chunk * ldp_n + n0 + t] = cs;
}

// C[k, n] = sum over chunks of the partials, in chunk order.
__global__ void tn_reduce(const float* __restrict__ part, int64_t n_chunks, int64_t ldp_k, int64_t ldp_n,
                          int64_t k1, int64_t k1p, int64_t k2, int64_t N, float* __restrict__ C, int64_t ldc,
                          const float* __restrict__ part_cs, float* __restrict__ colsum) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t rows = k1 + k2;
    if (idx < rows * N) {
        const int64_t k = idx / N, n = idx % N;
        const int64_t kv = k < k1 ? k : k1p + (k - k1);
        float s = 0.f;
        for (int64_t c = 0; c < n_chunks; ++c) s += part[(c * ldp_k + kv) * ldp_n + n];
        C[k * ldc + n] = s;
    }
    if (colsum && idx < N) {
        float s = 0.f;
        for (int64_t c = 0; c < n_chunks; ++c) s += part_cs[c * ldp_n + idx];
        colsum[idx] = s;
    }
}

// ---- packing of B -----------------------------------------------------------------
template <class T>
__global__ void pack_kernel(PackSrc src, int64_t k1, int64_t k1p, int64_t k2, int64_t Kt, NLayout nl,
                            int64_t n_pad, T* __restrict__ Bp) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= n_pad * Kt) return;
    const int64_t n = idx / Kt, k = idx % Kt;
    int s, tt;
    int64_t kk, nn;
    bool ok = true;
    if (k < k1p) { s = 0; kk = k; ok = kk < k1; }
    else { s = 1; kk = k - k1p; ok = kk < k2; }
    if (nl.n1 == 0 || n < nl.nsplit) { tt = 0; nn = n; ok = ok && nn < nl.n0; }
    else { tt = 1; nn = n - nl.nsplit; ok = ok && nn < nl.n1; }
    T v = from_f32<T>(0.f);
    if (ok && src.p[s][tt]) v = static_cast<const T*>(src.p[s][tt])[kk * src.sk[s][tt] + nn * src.sn[s][tt]];
    Bp[idx] = v;
}

// ---- ReLU mask ------------------------------------------------------------------------
template <class T>
__global__ void relu_mask_kernel(int64_t M, int64_t C, int64_t N, const T* __restrict__ G, int64_t ldg,
                                 const T* __restrict__ Y, int64_t ldy, T* __restrict__ out, int64_t ldo) {
    constexpr int V = Vec<T>::N;
    const int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (q >= M * C) return;
    const int64_t r = q / C, c0 = (q % C) * V;
    uint4 g = *reinterpret_cast<const uint4*>(G + r * ldg + c0);
    const uint4 y = *reinterpret_cast<const uint4*>(Y + r * ldy + c0);
    g = apply_mask<T>(g, y);
    const int n = static_cast<int>(min<int64_t>(V, N - c0));
    if (n == V) {
        *reinterpret_cast<uint4*>(out + r * ldo + c0) = g;
    } else {
        const uint32_t w[4] = {g.x, g.y, g.z, g.w};
        for (int e = 0; e < n; ++e) {
            if constexpr (V == 4) {
                reinterpret_cast<uint32_t*>(out + r * ldo + c0)[e] = w[e];
            } else {
                reinterpret_cast<uint16_t*>(out + r * ldo + c0)[e] =
                    static_cast<uint16_t>((e & 1) ? (w[e / 2] >> 16) : (w[e / 2] & 0xffffu));
            }
        }
    }
}

template <class T>
sag_status nn_typed(int64_t M, int64_t N, const GemmA& A, const void* Bp, sag_dtype dt, void* C, int64_t ldc,
                    const Epilogue& epi, hipStream_t s) {
    AOperand<T> ao = make_aop<T>(A, M, dt);
    const int64_t Kt = k_total(A.k1, A.a2 ? A.k2 : 0, dt);
    EpiT<T> e{static_cast<T*>(C), ldc, static_cast<T*>(epi.pre), static_cast<const T*>(epi.addend),
              epi.ld_add, epi.addend ? epi.n_add : 0, epi.bias, epi.relu};
    const int64_t mblk = cdiv(M, kBM);
    const T* B = static_cast<const T*>(Bp);
    if (N <= 64) {
        const int64_t nblk = cdiv(N, 64);
        gemm_nn<T, 64><<<dim3(static_cast<unsigned>(mblk * nblk)), 256, 0, s>>>(ao, B, Kt, N, nblk, e);
    } else if (N <= 128) {
        const int64_t nblk = cdiv(N, 128);
        gemm_nn<T, 128><<<dim3(static_cast<unsigned>(mblk * nblk)), 256, 0, s>>>(ao, B, Kt, N, nblk, e);
    } else {
        const int64_t nblk = cdiv(N, 256);
        gemm_nn<T, 256><<<dim3(static_cast<unsigned>(mblk * nblk)), 256, 0, s>>>(ao, B, Kt, N, nblk, e);
    }
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

struct TnPlan {
    int bnt;
    int64_t n_ktile, n_ntile, n_chunks, rows_per_chunk, ldp_k, ldp_n;
};

// The chunk count depends on M only (so workspace sizes grow with K and N):
// chunks of at least 256 rows, at most 512 chunks.
TnPlan tn_plan(int64_t M, int64_t Kv, int64_t N, sag_dtype dt) {
    TnPlan p;
    p.bnt = N <= 64 ? 64 : 128;
    p.n_ktile = cdiv(Kv > 0 ? Kv : 1, kBKT);
    p.n_ntile = cdiv(N > 0 ? N : 1, p.bnt);
    const int64_t ms = dt == SAG_BF16 ? 32 : 16;
    const int64_t m = M > 0 ? M : 1;
    int64_t want = cdiv(m, 256);
    if (want > 512) want = 512;
    const int64_t rpc = round_up(cdiv(m, want), ms);
    p.rows_per_chunk = rpc;
    p.n_chunks = cdiv(m, rpc);
    p.ldp_k = p.n_ktile * kBKT;
    p.ldp_n = p.n_ntile * p.bnt;
    return p;
}

template <class T>
sag_status tn_typed(int64_t M, int64_t N, const GemmA& A, const void* B, int64_t ldb, const void* mask,
                    int64_t ldmask, float* C, int64_t ldc, float* colsum, sag_dtype dt, void* ws, size_t ws_bytes,
                    hipStream_t s) {
    AOperand<T> ao = make_aop<T>(A, M, dt);
    const int64_t k2 = A.a2 ? A.k2 : 0;
    const int64_t Kv = kp(A.k1, dt) + kp(k2, dt);
    TnPlan p = tn_plan(M, Kv, N, dt);
    Carver c(ws, ws_bytes);
    float* part = c.take<float>(p.n_chunks * p.ldp_k * p.ldp_n);
    float* pcs = c.take<float>(p.n_chunks * p.ldp_n);
    if (!c.fits()) return fail(SAG_E_WORKSPACE, "gemm_tn: workspace too small");
    const unsigned grid = static_cast<unsigned>(p.n_chunks * p.n_ktile * p.n_ntile);
    if (p.bnt == 64)
        gemm_tn<T, 64><<<grid, 256, 0, s>>>(ao, static_cast<const T*>(B), ldb, static_cast<const T*>(mask), ldmask, N,
                                            p.n_ktile, p.n_ntile, p.rows_per_chunk, part, p.ldp_k, p.ldp_n,
                                            colsum ? pcs : nullptr);
    else
        gemm_tn<T, 128><<<grid, 256, 0, s>>>(ao, static_cast<const T*>(B), ldb, static_cast<const T*>(mask), ldmask, N,
                                             p.n_ktile, p.n_ntile, p.rows_per_chunk, part, p.ldp_k, p.ldp_n,
                                             colsum ? pcs : nullptr);
    SAG_LAUNCH_CHECK();
    const int64_t total = (A.k1 + k2) * N;
    const int64_t work = total > N ? total : N;
    tn_reduce<<<dim3(static_cast<unsigned>(cdiv(work, 256))), 256, 0, s>>>(
        part, p.n_chunks, p.ldp_k, p.ldp_n, A.k1, kp(A.k1, dt), k2, N, C, ldc, pcs, colsum);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace

size_t packed_b_bytes(int64_t k1, int64_t k2, int64_t n_total, sag_dtype dt) {
    return static_cast<size_t>(round_up(n_total > 0 ? n_total : 1, kNPad) * k_total(k1, k2, dt) * elt_size(dt));
}

sag_status pack_b(const PackSrc& src, int64_t k1, int64_t k2, const NLayout& nl, sag_dtype dt, void* Bp,
                  hipStream_t s) {
    const int64_t Kt = k_total(k1, k2, dt);
    const int64_t n_pad = round_up(nl.total() > 0 ? nl.total() : 1, kNPad);
    const int64_t total = n_pad * Kt;
    TraceScope trace(trace_enabled() ? shape_name("pack_b", dt == SAG_BF16 ? "bf16" : "f32", k1 + k2, nl.total(), 0)
                                     : std::string(),
                     s, elt_size(dt) * ((k1 + k2) * nl.total() + total), 0);
    const dim3 grid(static_cast<unsigned>(cdiv(total, 256)));
    if (dt == SAG_BF16)
        pack_kernel<uint16_t><<<grid, 256, 0, s>>>(src, k1, kp(k1, dt), k2, Kt, nl, n_pad, static_cast<uint16_t*>(Bp));
    else
        pack_kernel<float><<<grid, 256, 0, s>>>(src, k1, kp(k1, dt), k2, Kt, nl, n_pad, static_cast<float*>(Bp));
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

sag_status gemm_run(int64_t M, int64_t N, const GemmA& A, const void* Bp, sag_dtype dt, void* C, int64_t ldc,
                    const Epilogue& epi, hipStream_t s) {
    if (M == 0 || N == 0) return SAG_OK;
    const int64_t K = A.k1 + (A.a2 ? A.k2 : 0), e = elt_size(dt);
    const int64_t bytes = e * (M * K + K * N + M * N * (epi.pre ? 2 : 1)) + (A.mask ? e * M * A.k1 : 0) +
                          (epi.addend ? e * epi.n_add * N : 0);
    TraceScope trace(trace_enabled() ? shape_name("gemm_nn", dt == SAG_BF16 ? "bf16" : "f32", M, K, N) : std::string(),
                     s, bytes, 2 * M * K * N);
    if (dt == SAG_BF16) return nn_typed<uint16_t>(M, N, A, Bp, dt, C, ldc, epi, s);
    return nn_typed<float>(M, N, A, Bp, dt, C, ldc, epi, s);
}

size_t gemm_tn_ws_bytes(int64_t M, int64_t K, int64_t N, sag_dtype dt) {
    // K here is the padded virtual K (k1p + k2p) or an upper bound of it
    TnPlan p = tn_plan(M, K, N, dt);
    Carver c(nullptr, 0);
    c.take<float>(p.n_chunks * p.ldp_k * p.ldp_n);
    c.take<float>(p.n_chunks * p.ldp_n);
    return c.used();
}

sag_status gemm_tn_run(int64_t M, int64_t N, const GemmA& A, const void* B, int64_t ldb, const void* mask,
                       int64_t ldmask, float* C, int64_t ldc, float* colsum, sag_dtype dt, void* ws,
                       size_t ws_bytes, hipStream_t s) {
    if (N == 0) return SAG_OK;
    const int64_t K = (A.a1 ? A.k1 : 0) + (A.a2 ? A.k2 : 0), e = elt_size(dt);
    const int64_t bytes = e * (M * K + M * N * (mask ? 2 : 1)) + 4 * (K * N + (colsum ? N : 0));
    TraceScope trace(trace_enabled() ? shape_name("gemm_tn", dt == SAG_BF16 ? "bf16" : "f32", M, K, N) : std::string(),
                     s, bytes, 2 * M * K * N);
    if (dt == SAG_BF16)
        return tn_typed<uint16_t>(M, N, A, B, ldb, mask, ldmask, C, ldc, colsum, dt, ws, ws_bytes, s);
    return tn_typed<float>(M, N, A, B, ldb, mask, ldmask, C, ldc, colsum, dt, ws, ws_bytes, s);
}

sag_status relu_mask_run(int64_t M, int64_t N, const void* G, int64_t ldg, const void* Y, int64_t ldy, void* out,
                         int64_t ldo, sag_dtype dt, hipStream_t s) {
    if (M == 0 || N == 0) return SAG_OK;
    TraceScope trace(trace_enabled() ? shape_name("relu_mask", dt == SAG_BF16 ? "bf16" : "f32", M, N, 0) : std::string(),
                     s, 3 * elt_size(dt) * M * N, 0);
    const int64_t C = cdiv(N, vec_elems(dt));
    const dim3 grid(static_cast<unsigned>(cdiv(M * C, 256)));
    if (dt == SAG_BF16)
        relu_mask_kernel<uint16_t><<<grid, 256, 0, s>>>(M, C, N, static_cast<const uint16_t*>(G), ldg,
                                                        static_cast<const uint16_t*>(Y), ldy,
                                                        static_cast<uint16_t*>(out), ldo);
    else
        relu_mask_kernel<float><<<grid, 256, 0, s>>>(M, C, N, static_cast<const float*>(G), ldg,
                                                     static_cast<const float*>(Y), ldy, static_cast<float*>(out), ldo);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace sag

// ---- public entry points -------------------------------------------------------------
using namespace sag;

namespace {

sag_status check_gemm_a(const char* who, int64_t M, const void* A1, int64_t lda1, int64_t K1, const void* A2,
                        int64_t lda2, int64_t K2, const void* mask, int64_t ldmask, sag_dtype dt) {
    if (M < 0 || K1 < 0 || K2 < 0) return fail(SAG_E_INVALID, std::string(who) + ": negative size");
    SAG_TRY(check_dense("gemm A1", A1, M, K1, lda1, dt));
    if (A2 || K2) SAG_TRY(check_dense("gemm A2", A2, M, K2, lda2, dt));
    if (mask) SAG_TRY(check_dense("gemm mask", mask, M, K1, ldmask, dt));
    return SAG_OK;
}

}  // namespace

extern "C" size_t sag_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N, sag_dtype dt) {
    (void)M;
    if (K < 0 || N < 0) return 0;
    // two K blocks pad K by at most two vectors
    return packed_b_bytes(K + 2 * vec_elems(dt), 0, N, dt);
}

extern "C" sag_status sag_gemm(int64_t M, int64_t N, const void* A1, int64_t lda1, int64_t K1, const void* A2,
                               int64_t lda2, int64_t K2, const void* mask, int64_t ldmask, const void* B,
                               int64_t ldb, int trans_b, const float* bias, const void* addend, int64_t ld_add,
                               int relu, void* C, void* C_pre, int64_t ldc, sag_dtype dt, void* ws, size_t ws_bytes,
                               void* stream) {
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "gemm: bad dtype");
    if (N < 0) return fail(SAG_E_INVALID, "gemm: negative N");
    SAG_TRY(check_gemm_a("gemm", M, A1, lda1, K1, A2, lda2, K2, mask, ldmask, dt));
    const int64_t K = K1 + (A2 ? K2 : 0);
    if (K > 0 && N > 0 && !B) return fail(SAG_E_INVALID, "gemm: null B");
    if (ldb < (trans_b ? K : N)) return fail(SAG_E_INVALID, "gemm: ldb too small");
    SAG_TRY(check_dense("gemm C", C, M, N, ldc, dt));
    if (C_pre) SAG_TRY(check_dense("gemm C_pre", C_pre, M, N, ldc, dt));
    if (addend) SAG_TRY(check_dense("gemm addend", addend, M, N, ld_add, dt));
    if (ws_bytes < packed_b_bytes(K1, A2 ? K2 : 0, N, dt) || !ws) return fail(SAG_E_WORKSPACE, "gemm: workspace too small");
    hipStream_t s = static_cast<hipStream_t>(stream);
    PackSrc src;
    const int64_t sk = trans_b ? 1 : ldb, sn = trans_b ? ldb : 1;
    src.p[0][0] = B;
    src.sk[0][0] = sk;
    src.sn[0][0] = sn;
    if (A2) {
        const int64_t off = K1 * (trans_b ? 1 : ldb);
        src.p[1][0] = static_cast<const char*>(B) + off * elt_size(dt);
        src.sk[1][0] = sk;
        src.sn[1][0] = sn;
    }
    NLayout nl;
    nl.n0 = N;
    nl.nsplit = N;
    SAG_TRY(pack_b(src, K1, A2 ? K2 : 0, nl, dt, ws, s));
    GemmA a;
    a.a1 = A1; a.lda1 = lda1; a.k1 = K1; a.m1 = M;
    a.a2 = A2; a.lda2 = lda2; a.k2 = A2 ? K2 : 0;
    a.mask = mask; a.ldmask = ldmask;
    Epilogue e;
    e.bias = bias;
    e.addend = addend;
    e.ld_add = ld_add;
    e.n_add = addend ? M : 0;
    e.relu = relu;
    e.pre = C_pre;
    return gemm_run(M, N, a, ws, dt, C, ldc, e, s);
}

extern "C" size_t sag_gemm_tn_workspace_bytes(int64_t M, int64_t K, int64_t N, sag_dtype dt) {
    if (M < 0 || K < 0 || N < 0) return 0;
    // two blocks pad K by at most two vectors
    return gemm_tn_ws_bytes(M, K + 2 * vec_elems(dt), N, dt);
}

extern "C" sag_status sag_gemm_tn(int64_t M, int64_t N, const void* A1, int64_t lda1, int64_t K1, const void* A2,
                                  int64_t lda2, int64_t K2, const void* B, int64_t ldb, const void* mask,
                                  int64_t ldmask, float* C, int64_t ldc, float* colsum, sag_dtype dt, void* ws,
                                  size_t ws_bytes, void* stream) {
    if (dt != SAG_F32 && dt != SAG_BF16) return fail(SAG_E_INVALID, "gemm_tn: bad dtype");
    if (N < 0) return fail(SAG_E_INVALID, "gemm_tn: negative N");
    SAG_TRY(check_gemm_a("gemm_tn", M, A1, lda1, K1, A2, lda2, K2, nullptr, 0, dt));
    SAG_TRY(check_dense("gemm_tn B", B, M, N, ldb, dt));
    if (mask) SAG_TRY(check_dense("gemm_tn mask", mask, M, N, ldmask, dt));
    const int64_t K = K1 + (A2 ? K2 : 0);
    if (K > 0 && N > 0 && (!C || ldc < N)) return fail(SAG_E_INVALID, "gemm_tn: bad C");
    if (ws_bytes < sag_gemm_tn_workspace_bytes(M, K, N, dt) || !ws) return fail(SAG_E_WORKSPACE, "gemm_tn: workspace too small");
    GemmA a;
    a.a1 = A1; a.lda1 = lda1; a.k1 = K1; a.m1 = M;
    a.a2 = A2; a.lda2 = lda2; a.k2 = A2 ? K2 : 0;
    return gemm_tn_run(M, N, a, B, ldb, mask, ldmask, C, ldc, colsum, dt, ws, ws_bytes,
                       static_cast<hipStream_t>(stream));
}
