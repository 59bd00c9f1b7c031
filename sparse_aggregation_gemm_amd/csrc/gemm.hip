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
#include <type_traits>

#include "ops.h"
#include "trace.h"

namespace sag {

// Compute units of the current device (api.cpp), queried once per process.
int device_cus();

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Calls f(std::integral_constant<int, I>) for I in [B, E): register arrays
// indexed by I stay in registers however large the body is.
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kNPad = 256;   // N of a packed B is padded to this

inline int64_t kp(int64_t k, sag_dtype dt) { return round_up(k, vec_elems(dt)); }
// K blocks of the NN product are padded to whole 128-byte chunks (64 bf16,
// 32 fp32: four MFMA k-steps), so that every chunk lies inside one block.
inline int64_t kchunk(sag_dtype dt) { return dt == SAG_BF16 ? 64 : 32; }
inline int64_t kpc(int64_t k, sag_dtype dt) { return round_up(k, kchunk(dt)); }
// K of a packed B: a multiple of four chunks once it holds four, else of
// two (the NN kernel keeps that many chunks in flight).
inline int64_t k_total(int64_t k1, int64_t k2, sag_dtype dt) {
    const int64_t kv = kpc(k1, dt) + kpc(k2, dt);
    const int64_t c = kchunk(dt);
    return kv >= 4 * c ? round_up(kv, 4 * c) : round_up(kv, 2 * c);
}

// ---- element tricks on 16-byte vectors ---------------------------------------------

// Element-wise select of 16-byte vectors (a ?: on the vector class can be
// lowered through private memory).
__device__ __forceinline__ uint4 sel(bool c, const uint4& x, const uint4& y) {
    return make_uint4(c ? x.x : y.x, c ? x.y : y.y, c ? x.z : y.z, c ? x.w : y.w);
}

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

// The block operand [A1 | A2] seen through "virtual" columns: A1 occupies
// columns [0, k1p), A2 [k1p, k1p + k2p) (each padded to whole 16-byte
// vectors); anything else reads as zero.  Loading is split in two so that
// loads can be issued far ahead of their use without waiting: addr() gives
// an address that is always valid (out-of-range requests point at `safe`),
// and fix() zeroes what lies outside the operand once the data is used.
template <class T>
struct AOperand {
    const T* a1;
    int64_t lda1, k1, m1, k1p;
    const T* a2;
    int64_t lda2, k2, k2p;
    const T* mask;
    int64_t ldmask;
    int64_t M;
    const T* safe;   // any valid 16-byte aligned address

    // (a column in a block's padding is clamped to the block's last vector:
    // the row pitch covers that vector, so even the last row stays inside
    // the operand; fix() zeroes the values)
    static __device__ __forceinline__ int64_t last_vec(int64_t k) { return (k + Vec<T>::N - 1) / Vec<T>::N * Vec<T>::N - Vec<T>::N; }
    __device__ __forceinline__ const uint4* addr(int64_t r, int64_t k0) const {
        const T* p = safe;
        if (r < M) {
            if (k0 < k1p) {
                const int64_t last = last_vec(k1);
                if (r < m1) p = a1 + r * lda1 + (k0 < last ? k0 : last);
            } else if (k0 < k1p + k2p) {
                const int64_t kk = k0 - k1p, last = last_vec(k2);
                p = a2 + r * lda2 + (kk < last ? kk : last);
            }
        }
        return reinterpret_cast<const uint4*>(p);
    }
    __device__ __forceinline__ const uint4* mask_addr(int64_t r, int64_t k0) const {
        const T* p = safe;
        const int64_t last = last_vec(k1);
        if (mask && r < M && r < m1 && k0 < k1p) p = mask + r * ldmask + (k0 < last ? k0 : last);
        return reinterpret_cast<const uint4*>(p);
    }
    __device__ __forceinline__ uint4 fix(uint4 v, int64_t r, int64_t k0) const {
        const bool in1 = k0 < k1p, in2 = !in1 && k0 < k1p + k2p;
        const int n = in1 ? static_cast<int>(k1 - k0) : static_cast<int>(k2 - (k0 - k1p));
        const bool ok = r < M && ((in1 && r < m1) || in2);
        return sel(ok, keep_first<T>(v, n), make_uint4(0, 0, 0, 0));
    }
    __device__ __forceinline__ uint4 fix_masked(uint4 v, uint4 m, int64_t r, int64_t k0) const {
        v = fix(v, r, k0);
        return sel(mask && k0 < k1p, apply_mask<T>(v, m), v);
    }
    // ---- streaming access used by the NN kernel ----
    // Row pointers of row r (clamped to a valid row: rows >= M only feed
    // outputs that are never stored).
    __device__ __forceinline__ void row_ptrs(int64_t r, const T*& p1, const T*& p2) const {
        const int64_t rc = r < M ? r : M - 1;
        p1 = a1 ? a1 + (rc < m1 ? rc : m1 - 1) * lda1 : safe;
        p2 = a2 ? a2 + rc * lda2 : p1;
    }
    // Address of the vector at virtual column k0, clamped into the operand.
    __device__ __forceinline__ const uint4* stream_addr(const T* p1, const T* p2, int64_t k0) const {
        const int64_t last = k1p + k2p - Vec<T>::N;
        const int64_t kc = k0 < last ? k0 : last;
        return reinterpret_cast<const uint4*>(kc < k1p ? p1 + kc : p2 + (kc - k1p));
    }
    // True when the k-range [kb, kb + span) holds a column that must read as
    // zero: the ragged tail of a block or anything past the operand.
    __device__ __forceinline__ bool needs_fix(int64_t kb, int64_t span) const {
        return (kb + span > k1 && kb < k1p) || (kb + span > k1p + k2);
    }
    // one-shot load (used where the value is needed at once)
    __device__ __forceinline__ uint4 load(int64_t r, int64_t k0) const {
        const uint4 v = *addr(r, k0);
        return mask ? fix_masked(v, *mask_addr(r, k0), r, k0) : fix(v, r, k0);
    }
};

// pad: the K padding of each block (16-byte vectors for TN, k-steps for NN).
template <class T>
AOperand<T> make_aop(const GemmA& A, int64_t M, sag_dtype dt, const void* safe, int64_t pad) {
    AOperand<T> o;
    o.a1 = static_cast<const T*>(A.a1);
    o.lda1 = A.lda1;
    o.k1 = A.a1 ? A.k1 : 0;
    o.m1 = A.a1 ? (A.m1 > 0 ? A.m1 : M) : 0;
    o.k1p = A.a1 ? round_up(A.k1, pad) : 0;
    o.a2 = static_cast<const T*>(A.a2);
    o.lda2 = A.lda2;
    o.k2 = A.a2 ? A.k2 : 0;
    o.k2p = A.a2 ? round_up(A.k2, pad) : 0;
    o.mask = static_cast<const T*>(A.mask);
    o.ldmask = A.ldmask;
    o.M = M;
    o.safe = static_cast<const T*>(safe);
    return o;
}

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

// Stores n <= 4 consecutive values (4 as one vector: 8 bytes of bf16 or 16
// bytes of fp32; p is aligned for that when n == 4).
template <class T>
__device__ __forceinline__ void store4(T* p, const float* y, int n) {
    if (n == 4) {
        if constexpr (sizeof(T) == 2) {
            const uint32_t lo = uint32_t(f32_to_bf16(y[0])) | (uint32_t(f32_to_bf16(y[1])) << 16);
            const uint32_t hi = uint32_t(f32_to_bf16(y[2])) | (uint32_t(f32_to_bf16(y[3])) << 16);
            *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
        } else {
            *reinterpret_cast<float4*>(p) = make_float4(y[0], y[1], y[2], y[3]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (t < n) p[t] = from_f32<T>(y[t]);
    }
}

// ---- NN ------------------------------------------------------------------------------
// C = A B with M huge and K, N small (the layer's transform and input
// gradient).  A workgroup keeps its BN columns of the packed B (all of K)
// in LDS for its whole life; each of its eight wavefronts walks 32-row
// blocks of A.  A is read in chunks of 128 bytes of k per row with eight
// lanes per row, so every load instruction fetches four whole cache lines;
// the chunk goes through a per-wavefront LDS tile into the MFMA operand
// layout, PD chunks ahead in registers.  The results go back through the
// same tile so that C is written in whole lines as well.  The tile and the
// B slice XOR-swizzle their 16-byte units so that row-strided fragment
// reads do not collide in banks.  The K blocks
// A1 and A2 are padded to whole chunks in the packed B, so each chunk comes
// from one block and only the last chunk of a block needs zeroing.
//
// The MFMAs compute transposed blocks, C^T = B^T A^T: B supplies the first
// operand and A the second, so lane l accumulates row l%32 of a 32x32 block
// of C and register r holds column 8*(r/4) + 4*(l/32) + r%4.  bf16: unit
// h of a k-step holds its k 8h..8h+7, the operand of one 32x32x16 MFMA.
// fp32: unit h holds k 4h..4h+3 of the k-step; four 32x32x2 MFMAs pair
// k+q with k+4+q (B is stored with the same pairing).
constexpr int kNnWaves = 8;
constexpr int kNnRows = 32;                       // rows of a wavefront block
constexpr int kNnTile = kNnRows * 128;            // bytes of a wavefront's tile

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// LDS swizzles, free of bank conflicts whether a 16-byte access of 16 lanes
// is served from a 256-byte or (8 lanes) from a 128-byte window:
// the 16-byte unit of row r of a 128-byte-row tile is XORed with asw(r),
// the unit (0/1) of column n of the 32-byte-unit B slice with bsw(n).
__device__ __forceinline__ int asw(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int bsw(int n) { return ((n >> 2) ^ (n >> 3)) & 1; }

// Two fp32 values as packed bf16 (round to nearest even, one instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ReLU on eight packed bf16 values: zeroes the negative ones, leaving -0 and
// NaN as they are (as max(y, 0) on the fp32 value before rounding would).
__device__ __forceinline__ uint4 relu_bf16x8(uint4 v) {
    uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const uint32_t b = (q & 1) ? (wv[q / 2] >> 16) : (wv[q / 2] & 0xffffu);
        const uint32_t mag = b & 0x7fffu;
        if ((b & 0x8000u) && mag != 0u && mag <= 0x7f80u) wv[q / 2] &= (q & 1) ? 0x0000ffffu : 0xffff0000u;
    }
    return make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

template <class T, int BN, bool MASK, int PD>
__global__ __launch_bounds__(kNnWaves * 64, 1) void gemm_nn(AOperand<T> A, const T* __restrict__ Bp, int64_t Kt,
                                                             int64_t N, int64_t n_nblk, int64_t n_mgroups,
                                                             int64_t n_blk, EpiT<T> e,
                                                             const float* __restrict__ bias) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    constexpr int V = Vec<T>::N;                  // elements per 16-byte unit
    constexpr int CKE = 128 / static_cast<int>(sizeof(T));   // elements per chunk (4 k-steps)
    constexpr int NB = BN / 32;
    constexpr int LPR = kNnRows / 8;              // loads per lane per chunk
    // epilogue groups: 64 columns of bf16 or 32 of fp32 make one 128-byte row
    constexpr int GB = (sizeof(T) == 2 && NB % 2 == 0) ? 2 : 1;   // 32-column blocks per group
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int rr = lane >> 3, u = lane & 7;       // chunk load: sub-row, 16-byte unit
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t nb = tile % n_nblk, mg = tile / n_nblk;
    const int64_t n0 = nb * BN;
    unsigned char* Bs = lds_raw;                  // [k-step][BN] 32-byte units
    unsigned char* At = lds_raw + static_cast<size_t>(BN) * Kt * sizeof(T) + wave * kNnTile;
    {
        // unit w (0/1) of k-step ks of column n sits at (ks*BN + n)*32 + 16*(w ^ bsw(n))
        const int64_t kvec = Kt / V;
        for (int64_t q = threadIdx.x; q < BN * kvec; q += kNnWaves * 64) {
            const int64_t n = q / kvec, c = q % kvec;
            const int64_t ks = c >> 1, w = c & 1;
            *reinterpret_cast<uint4*>(Bs + (ks * BN + n) * 32 + ((w ^ bsw(static_cast<int>(n))) << 4)) =
                *reinterpret_cast<const uint4*>(Bp + (n0 + n) * Kt + c * V);
        }
    }
    __syncthreads();
    const int64_t stride = n_mgroups * kNnWaves;
    int64_t b = mg * kNnWaves + wave;
    if (b >= n_blk) return;
    const int nch = static_cast<int>(Kt / CKE);   // a multiple of PD
    const int nc1 = static_cast<int>(A.k1p / CKE);
    const int64_t last1 = (A.k1 + V - 1) / V * V - V, last2 = (A.k2 + V - 1) / V * V - V;
    const int64_t m1c = A.m1 > 0 ? A.m1 - 1 : 0, mc = A.M - 1;
    // source of chunk c: block 1 for c < nc1, else block 2 (or, past both
    // blocks, block 1 clamped: read and then zeroed)
    struct Src {
        const T* base;
        int64_t ld, lim, col;
    };
    auto src_of = [&](int c) -> Src {
        Src s;
        const bool p1 = c < nc1 || !A.a2;
        const int64_t cc = static_cast<int64_t>(p1 ? c : c - nc1) * CKE + u * V;
        const int64_t last = p1 ? last1 : last2;
        s.base = p1 ? A.a1 : A.a2;
        s.ld = p1 ? A.lda1 : A.lda2;
        s.lim = p1 ? m1c : mc;
        s.col = cc < last ? cc : last;
        return s;
    };
    uint4 ra[PD][LPR], rm[MASK ? PD : 1][LPR];
    auto issue = [&](auto slot_c, int64_t blk, int c) {
        constexpr int slot = decltype(slot_c)::value;
        const Src s = src_of(c);
        const int64_t row0 = blk * kNnRows + rr;
        // the mask of a chunk past block 1 is read (clamped) but not used
        const int64_t mcol = s.col < last1 ? s.col : last1;
#pragma unroll
        for (int i = 0; i < LPR; ++i) {
            const int64_t r = row0 + 8 * i < s.lim ? row0 + 8 * i : s.lim;
            ra[slot][i] = *reinterpret_cast<const uint4*>(s.base + r * s.ld + s.col);
            if constexpr (MASK) {
                const int64_t rmk = row0 + 8 * i < m1c ? row0 + 8 * i : m1c;
                rm[slot][i] = *reinterpret_cast<const uint4*>(A.mask + rmk * A.ldmask + mcol);
            }
        }
    };
    // fragment read offsets: A row l32, unit 2s + h; B column l32 of a block, unit h
    int aoff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[s] = l32 * 128 + (((2 * s + h) ^ asw(l32)) << 4);
    const int boff = l32 * 32 + ((h ^ bsw(l32)) << 4);
    static_for<0, PD>([&](auto sc) { issue(sc, b, decltype(sc)::value); });
    for (;;) {
        f32x16_t acc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
        const int64_t b_next = b + stride;
        const int64_t b_end = b * kNnRows + kNnRows;
        const bool edge_rows = b_end > A.M || (A.a1 && b_end > A.m1);
        for (int c0 = 0; c0 < nch; c0 += PD) {
            static_for<0, PD>([&](auto sc) {
                constexpr int slot = decltype(sc)::value;
                const int c = c0 + slot;
                const bool p1 = c < nc1 || !A.a2;
                const int64_t kpart = p1 ? A.k1 : A.k2;
                const int64_t cc = static_cast<int64_t>(p1 ? c : c - nc1) * CKE;
                const bool edge_k = cc + CKE > kpart;
#pragma unroll
                for (int i = 0; i < LPR; ++i) {
                    uint4 v = ra[slot][i];
                    if constexpr (MASK) {
                        if (c < nc1) v = apply_mask<T>(v, rm[slot][i]);
                    }
                    if (edge_rows || edge_k) {
                        const int64_t row = b * kNnRows + 8 * i + rr;
                        const bool ok = row < A.M && (!p1 || !A.a1 || row < A.m1);
                        v = sel(ok, keep_first<T>(v, static_cast<int>(kpart - cc - u * V)), make_uint4(0, 0, 0, 0));
                    }
                    *reinterpret_cast<uint4*>(At + (8 * i + rr) * 128 + ((u ^ asw(8 * i + rr)) << 4)) = v;
                }
                int cn = c + PD;
                int64_t bn = b;
                if (cn >= nch) {
                    cn -= nch;
                    bn = b_next;
                }
                issue(sc, bn, cn);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const uint4 a = *reinterpret_cast<const uint4*>(At + aoff[s]);
                    const unsigned char* bk = Bs + static_cast<int64_t>(c * 4 + s) * BN * 32 + boff;
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const uint4 bv = *reinterpret_cast<const uint4*>(bk + j * 32 * 32);
                        if constexpr (sizeof(T) == 2) {
                            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv),
                                                                              __builtin_bit_cast(bf16x8_t, a),
                                                                              acc[j], 0, 0, 0);
                        } else {
                            const f32x4_t bb = __builtin_bit_cast(f32x4_t, bv);
                            const f32x4_t aa = __builtin_bit_cast(f32x4_t, a);
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bb[q], aa[q], acc[j], 0, 0, 0);
                        }
                    }
                }
            });
        }
        // ---- epilogue: per group of GB column blocks, bias (+ addend), then
        // Y_pre and/or the (ReLU'd) output through the tile as whole rows
        const int64_t row = b * kNnRows + l32;
#pragma unroll
        for (int g = 0; g < NB / GB; ++g) {
            float y[GB][4][4];
#pragma unroll
            for (int jj = 0; jj < GB; ++jj) {
                const int j = g * GB + jj;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t cb = n0 + j * 32 + 8 * q;   // uniform: columns cb + 4h + t
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        float bv = 0.f;
                        if (bias) {
                            const float lo = cb + t < N ? bias[cb + t] : 0.f;
                            const float hi = cb + 4 + t < N ? bias[cb + 4 + t] : 0.f;
                            bv = h ? hi : lo;
                        }
                        y[jj][q][t] = acc[j][4 * q + t] + bv;
                    }
                    if (e.add && row < e.n_add) {
                        const int64_t col = cb + 4 * h;
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (col + t < N) y[jj][q][t] += to_f32(e.add[row * e.ld_add + col + t]);
                    }
                }
            }
            const int64_t gc0 = n0 + g * GB * 32;       // first column of the group
            // two passes when Y_pre is wanted: pre-activation, then output
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                T* dst;
                if (pass == 0) {
                    if (!e.pre) continue;
                    dst = e.pre;
                } else {
                    dst = e.c;
                    if (e.relu) {
#pragma unroll
                        for (int jj = 0; jj < GB; ++jj)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
#pragma unroll
                                for (int t = 0; t < 4; ++t) y[jj][q][t] = y[jj][q][t] < 0.f ? 0.f : y[jj][q][t];
                    }
                }
                // stage: row l32, columns jj*32 + 8q + 4h .. +3 of the group
#pragma unroll
                for (int jj = 0; jj < GB; ++jj) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if constexpr (sizeof(T) == 2) {
                            const uint32_t lo = pack_bf16x2(y[jj][q][0], y[jj][q][1]);
                            const uint32_t hi = pack_bf16x2(y[jj][q][2], y[jj][q][3]);
                            const int w = jj * 4 + q;     // 16-byte unit of the 128-byte row
                            *reinterpret_cast<uint2*>(At + l32 * 128 + ((w ^ asw(l32)) << 4) + h * 8) =
                                make_uint2(lo, hi);
                        } else {
                            const int w = 2 * q + h;
                            *reinterpret_cast<float4*>(At + l32 * 128 + ((w ^ asw(l32)) << 4)) =
                                make_float4(y[jj][q][0], y[jj][q][1], y[jj][q][2], y[jj][q][3]);
                        }
                    }
                }
                // whole rows back out: lane -> row 8i + rr, unit u
                constexpr int UNITS = GB * 32 * static_cast<int>(sizeof(T)) / 16;   // 16-byte units per row
#pragma unroll
                for (int i = 0; i < LPR; ++i) {
                    const int r = 8 * i + rr;
                    const int64_t grow = b * kNnRows + r;
                    if (u >= UNITS) continue;
                    const uint4 v = *reinterpret_cast<const uint4*>(At + r * 128 + ((u ^ asw(r)) << 4));
                    const int64_t col = gc0 + u * V;
                    if (grow >= A.M || col >= N) continue;
                    T* p = dst + grow * e.ldc + col;
                    if (col + V <= N) {
                        *reinterpret_cast<uint4*>(p) = v;
                    } else {
                        const int n = static_cast<int>(N - col);
                        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
                        for (int t = 0; t < n; ++t) {
                            if constexpr (sizeof(T) == 2)
                                p[t] = static_cast<T>((t & 1) ? (wv[t / 2] >> 16) : (wv[t / 2] & 0xffffu));
                            else
                                p[t] = __uint_as_float(wv[t]);
                        }
                    }
                }
            }
        }
        b = b_next;
        if (b >= n_blk) break;
    }
}

// ---- NN with the weights in registers (bf16) -----------------------------------------
// When K times the columns of a wavefront is at most 512 bf16 (K <= 512 and
// N <= 256, or K <= 256 and N <= 512), each of the eight wavefronts keeps
// the packed-B fragments of its output column blocks (blocks w and w + 8) in
// registers for the whole kernel: 16 bytes per lane per k-step and block.
// The workgroup then needs one LDS copy of a 32-row A tile for all N
// columns, so A is read from HBM once (the LDS-resident kernel above reads
// each A tile once per 128-column block).  Workgroups are persistent and
// walk the tiles: the whole-line loads of the next PF tiles sit in
// registers, the A tile is double-buffered in LDS (one barrier per tile),
// and each wavefront stages and stores its own 32 x 32 output blocks with no
// workgroup barrier.  Operand layout and epilogue as in gemm_nn (no addend).
constexpr int kRwWaves = 8;
constexpr int kRwRows = 32;
constexpr int kRwStage = 32 * (64 + 16);          // bytes of one wavefront's staged 32 x 32 block

template <int KS> constexpr int rw_atile() { return kRwRows * (KS * 32 + 16); }

template <int KS, int NBW, bool MASK, int PF, int WPE>
__global__ __launch_bounds__(kRwWaves * 64, WPE) void gemm_nn_rw(AOperand<uint16_t> A,
                                                               const uint16_t* __restrict__ Bp, int64_t Kt,
                                                               int64_t N, int NB, int64_t n_tiles,
                                                               EpiT<uint16_t> e, const float* __restrict__ bias) {
    using T = uint16_t;
    constexpr int KU = KS * 2;                        // 16-byte units of a tile row
    constexpr int UNITS = kRwRows * KU;
    constexpr int NT = kRwWaves * 64;
    constexpr int UPT = (UNITS + NT - 1) / NT;        // units per thread
    constexpr int PITCH = KU * 16 + 16;               // tile row pitch (bytes)
    constexpr int ATILE = rw_atile<KS>();
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    unsigned char* stage = lds_raw + 2 * ATILE + wave * NBW * kRwStage;
    // the bias of every column the workgroup writes (0 past N or without a
    // bias), copied to LDS once: per-lane global loads in the epilogue would
    // be issued after the next tiles' prefetch, and waiting for them would
    // drain that prefetch every tile
    float* bias_s = reinterpret_cast<float*>(lds_raw + 2 * ATILE + kRwWaves * NBW * kRwStage);
    const int64_t G = gridDim.x;
    int64_t t = blockIdx.x;
    if (t >= n_tiles) return;
    for (int n = tid; n < kRwWaves * NBW * 32; n += kRwWaves * 64) bias_s[n] = bias && n < N ? bias[n] : 0.f;

    uint4 w[NBW][KS];
    bool has[NBW];
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
        const int nb = wave + kRwWaves * j;
        has[j] = nb < NB;
        const T* col = Bp + static_cast<int64_t>(nb * 32 + l32) * Kt + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            w[j][ks] = has[j] ? *reinterpret_cast<const uint4*>(col + ks * 16) : make_uint4(0, 0, 0, 0);
    }

    uint4 ra[PF][UPT], rm[MASK ? PF : 1][UPT];
    // (no tile bound: rows past M load from a valid address, so every step
    // issues the same loads and the compiler's wait counts stay exact)
    auto issue = [&](auto slot_c, int64_t tile) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            const int64_t row = tile * kRwRows + u / KU;
            const int64_t k0 = static_cast<int64_t>(u % KU) * 8;
            ra[slot][i] = *A.addr(row, k0);
            if constexpr (MASK) rm[slot][i] = *A.mask_addr(row, k0);
        }
    };
    auto stash = [&](auto slot_c, int64_t tile, unsigned char* buf) __attribute__((always_inline)) {
        constexpr int slot = decltype(slot_c)::value;
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            const int r = u / KU, c = u % KU;
            const int64_t row = tile * kRwRows + r;
            uint4 v;
            if constexpr (MASK) v = A.fix_masked(ra[slot][i], rm[slot][i], row, static_cast<int64_t>(c) * 8);
            else v = A.fix(ra[slot][i], row, static_cast<int64_t>(c) * 8);
            *reinterpret_cast<uint4*>(buf + r * PITCH + c * 16) = v;
        }
    };
    auto compute = [&](int64_t tile, const unsigned char* buf) __attribute__((always_inline)) {
        f32x16_t acc[NBW];
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
        const unsigned char* arow = buf + l32 * PITCH + h * 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4*>(arow + ks * 32);
#pragma unroll
            for (int j = 0; j < NBW; ++j)
                if (has[j])
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w[j][ks]),
                                                                      __builtin_bit_cast(bf16x8_t, a), acc[j], 0, 0,
                                                                      0);
        }
        // this wavefront's blocks: bias, one rounding, staged as row l32,
        // columns 8q + 4h .. +3 of the block, then stored as 64-byte row pieces
#pragma unroll
        for (int j = 0; j < NBW; ++j) {
            if (!has[j]) continue;
            const int nb = wave + kRwWaves * j;
            unsigned char* st = stage + j * kRwStage;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 bv = *reinterpret_cast<const float4*>(bias_s + nb * 32 + 8 * q + 4 * h);
                const float y[4] = {acc[j][4 * q] + bv.x, acc[j][4 * q + 1] + bv.y, acc[j][4 * q + 2] + bv.z,
                                    acc[j][4 * q + 3] + bv.w};
                *reinterpret_cast<uint2*>(st + l32 * 80 + (8 * q + 4 * h) * 2) =
                    make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = (lane >> 2) + 16 * i, c = lane & 3;
                const int64_t grow = tile * kRwRows + r;
                const int64_t col = static_cast<int64_t>(nb) * 32 + c * 8;
                if (grow >= A.M || col >= N) continue;
                uint4 v = *reinterpret_cast<const uint4*>(st + r * 80 + c * 16);
                const int n = static_cast<int>(N - col < 8 ? N - col : 8);
#pragma unroll
                for (int pass = 0; pass < 2; ++pass) {
                    T* dst;
                    if (pass == 0) {
                        if (!e.pre) continue;
                        dst = e.pre;
                    } else {
                        dst = e.c;
                        if (e.relu) v = relu_bf16x8(v);
                    }
                    T* p = dst + grow * e.ldc + col;
                    if (n == 8) {
                        *reinterpret_cast<uint4*>(p) = v;
                    } else {
                        // a ragged last unit: whole 4-byte pairs, then the odd element
                        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                        for (int q = 0; q < 3; ++q)
                            if (2 * q + 1 < n) reinterpret_cast<uint32_t*>(p)[q] = wv[q];
                        if (n & 1) p[n - 1] = static_cast<T>(wv[n / 2] & 0xffffu);
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    };

    // Register slot s holds tile t + s*G at the start.  Step k computes tile
    // t_k from LDS buffer k % 2 after moving tile t_{k+1} into the other
    // buffer and refilling its slot with tile t_{k+1+PF}; one barrier ends
    // the step (every wavefront is then done with buffer k % 2 and tile
    // t_{k+1} is complete in the other).  Steps run in whole rounds of PF
    // with no exit inside a round; a step past the workgroup's last tile
    // computes zeros and stores nothing (its rows are >= M).
    const int64_t steps = (n_tiles - t + G - 1) / G;
    static_for<0, PF>([&](auto sc) __attribute__((always_inline)) { issue(sc, t + decltype(sc)::value * G); });
    stash(std::integral_constant<int, 0>{}, t, lds_raw);
    __syncthreads();
    issue(std::integral_constant<int, 0>{}, t + PF * G);
    int cur = 0;
    for (int64_t k = 0; k < steps; k += PF) {
        static_for<0, PF>([&](auto sc) __attribute__((always_inline)) {
            constexpr int nx = (decltype(sc)::value + 1) % PF;
            unsigned char* nbuf = lds_raw + (cur ^ 1) * ATILE;
            stash(std::integral_constant<int, nx>{}, t + G, nbuf);
            issue(std::integral_constant<int, nx>{}, t + (PF + 1) * G);
            compute(t, lds_raw + cur * ATILE);
            __syncthreads();
            cur ^= 1;
            t += G;
        });
    }
}


// Tiles in flight per workgroup: as many as the registers hold next to the
// weight fragments (every slot is live at once: the loop issues the same
// loads on every step, so the waits count exactly and never drain the
// prefetch); the masked 16-step kernel with two blocks per wavefront spills
// 12 bytes even at one tile and is still faster than with conditional
// loads.  WPE is the minimum of waves per
// SIMD handed to __launch_bounds__ (HIP's second argument counts waves per
// execution unit, not workgroups per CU): an 8-wave workgroup is 2 waves per
// SIMD, so 2 only caps the registers at 256.  The KS * NBW <= 8 kernel needs
// 110 registers and runs two workgroups per CU, as the occupancy query that
// sizes the grid reports; the others need 138-256 and run one.  Asking for 4
// (two workgroups) at K = 256 spills to scratch at every prefetch depth.
template <int KS, int NBW, bool MASK>
constexpr int rw_pf() { return KS * NBW >= 32 ? 1 : (KS * NBW >= 16 ? (MASK ? 2 : 3) : 6); }
template <int KS, int NBW, bool MASK>
constexpr int rw_wpe() { return KS * NBW <= 8 && !MASK ? 2 : 1; }

template <int KS, int NBW, bool MASK>
sag_status launch_nn_rw(const AOperand<uint16_t>& ao, const uint16_t* B, int64_t Kt, int64_t N,
                        const EpiT<uint16_t>& e, const float* bias, hipStream_t s) {
    constexpr int PF = rw_pf<KS, NBW, MASK>(), WPE = rw_wpe<KS, NBW, MASK>();
    const int NB = static_cast<int>(cdiv(N, 32));
    constexpr size_t lds = 2 * static_cast<size_t>(rw_atile<KS>()) + static_cast<size_t>(kRwWaves) * NBW * kRwStage +
                           static_cast<size_t>(kRwWaves) * NBW * 32 * sizeof(float);
    // (once per kernel instance: the initialisation of a function-local
    // static is thread-safe)
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gemm_nn_rw<KS, NBW, MASK, PF, WPE>), hipFuncAttributeMaxDynamicSharedMemorySize,
        131072);
    SAG_CHECK_HIP(attr);
    // persistent workgroups: exactly as many as are resident at once
    static const int per_cu = [] {
        int nb = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &nb, reinterpret_cast<const void*>(&gemm_nn_rw<KS, NBW, MASK, PF, WPE>), kRwWaves * 64, lds) ==
                       hipSuccess && nb > 0
                   ? nb
                   : 1;
    }();
    const int64_t n_tiles = cdiv(ao.M, kRwRows);
    int64_t grid = static_cast<int64_t>(device_cus()) * per_cu;
    if (grid > n_tiles) grid = n_tiles;
    gemm_nn_rw<KS, NBW, MASK, PF, WPE><<<dim3(static_cast<unsigned>(grid)), kRwWaves * 64, lds, s>>>(
        ao, B, Kt, N, NB, n_tiles, e, bias);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

// The register-resident kernel for bf16 without an addend when N > 128 and
// K * (columns per wavefront) <= 512; returns SAG_E_UNSUPPORTED otherwise
// (the caller then takes the LDS-resident kernel).
sag_status try_nn_rw(const AOperand<uint16_t>& ao, const uint16_t* B, int64_t Kt, int64_t N,
                     const EpiT<uint16_t>& e, const float* bias, hipStream_t s) {
    if (e.add) return SAG_E_UNSUPPORTED;
    const int64_t NB = cdiv(N, 32);
    // up to 128 columns the LDS-resident kernel reads A once as well, and
    // is faster at K = 256 (256 -> 128: 0.44 against 0.49 ms; 256 -> 64: 0.33
    // against 0.45), but not at K = 128 (128 -> 128: 0.36 against 0.24),
    // where this kernel runs two workgroups per CU
    if (NB <= 4 && (Kt != 128 || ao.mask)) return SAG_E_UNSUPPORTED;
    const int nbw = NB <= kRwWaves ? 1 : (NB <= 2 * kRwWaves ? 2 : 0);
    const bool m = ao.mask != nullptr;
    if (nbw == 1) {
        switch (Kt) {
            case 128: return m ? launch_nn_rw<8, 1, true>(ao, B, Kt, N, e, bias, s) : launch_nn_rw<8, 1, false>(ao, B, Kt, N, e, bias, s);
            case 256: return m ? launch_nn_rw<16, 1, true>(ao, B, Kt, N, e, bias, s) : launch_nn_rw<16, 1, false>(ao, B, Kt, N, e, bias, s);
            // (a mask at K = 512 would spill the weight fragments)
            case 512: return m ? SAG_E_UNSUPPORTED : launch_nn_rw<32, 1, false>(ao, B, Kt, N, e, bias, s);
            default: return SAG_E_UNSUPPORTED;
        }
    }
    if (nbw == 2) {
        switch (Kt) {
            case 128: return m ? launch_nn_rw<8, 2, true>(ao, B, Kt, N, e, bias, s) : launch_nn_rw<8, 2, false>(ao, B, Kt, N, e, bias, s);
            case 256: return m ? launch_nn_rw<16, 2, true>(ao, B, Kt, N, e, bias, s) : launch_nn_rw<16, 2, false>(ao, B, Kt, N, e, bias, s);
            default: return SAG_E_UNSUPPORTED;
        }
    }
    return SAG_E_UNSUPPORTED;
}

// ---- NN with A streamed through an LDS ring (bf16, no mask, no addend) -------------
// The weights stay in registers as in gemm_nn_rw (wavefront w owns the
// 32-column block w over all of K), but the 32-row tiles of A go from HBM
// straight into LDS with direct loads (global_load_lds_dwordx4: lane i of a
// wavefront writes bytes [16 i, 16 i + 16) of a 1 KB block at the address
// in M0), so registers no longer bound the prefetch depth: S slots, S - 1
// tiles in flight behind the one being multiplied.  In a slot, unit c (16
// bytes) of row r sits at position c ^ (r & 15), so the 32 rows that a
// wavefront reads at once spread over all banks.  Units past a block's
// columns, and rows past the operand, are loaded from a zero vector; the
// one unit of a block that is partly inside it is masked in LDS by the lane
// that loaded it, once per tile, so the MFMA loop has no branches and its
// LDS reads run a batch ahead of the products.
//
// Synchronisation: each wavefront waits for its own direct loads of the
// next tile with an explicit count, then the workgroup meets at a bare
// barrier (a fence would wait for every load in flight, draining the ring).
// The count is exact because every wavefront with a block issues at least
// kRgStores stores per tile (stores that fall outside C go to a sink) and
// nothing else touches vector memory in the loop; the empty asm statements
// keep the compiler from moving memory operations across these points.
constexpr int kRgWaves = 8;
constexpr int kRgRows = 32;
constexpr int kRgStores = 2;                     // C stores per tile and lane (two 16-row halves)

__device__ __attribute__((aligned(16))) uint4 g_ring_zero;                 // never written
__device__ __attribute__((aligned(16))) uint4 g_ring_sink[kRgWaves * 64];  // never read

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One direct load: 16 bytes per lane from g into LDS at lds + 16 * lane.  In
// asm rather than through the builtin: the compiler would otherwise make
// every later LDS read wait for the newest direct load (it cannot tell the
// ring slots apart), which would drain the ring at each step.  The load takes
// its LDS address from M0, a register the compiler reserves for itself, so
// the asm keeps M0's value in a scratch SGPR and puts it back after issuing
// the load (a wait state on each side of the load; no vector register is
// written).
__device__ __forceinline__ void lds_direct_load16(const void* g, uint32_t lds) {
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(g), "s"(lds)
        : "memory");
}

// s_waitcnt with vmcnt = N and lgkmcnt = 0 (expcnt not waited for); the
// immediate holds vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4)); }
__device__ __forceinline__ void mem_order() { asm volatile("" ::: "memory"); }

template <int KS, int S, bool PP, int WPE>
__global__ __launch_bounds__(kRgWaves * 64, WPE) void gemm_nn_ring(AOperand<uint16_t> A,
                                                                  const uint16_t* __restrict__ Bp, int64_t Kt,
                                                                  int64_t N, int NB, int64_t n_tiles,
                                                                  EpiT<uint16_t> e, const float* __restrict__ bias,
                                                                  int fixup) {
    using T = uint16_t;
    constexpr int U = KS * 2;                     // 16-byte units of a tile row
    constexpr int ROWB = U * 16;
    constexpr int SLOT = kRgRows * ROWB;          // = 1024 KS
    constexpr int IPW = SLOT / 1024 / kRgWaves;   // direct-load instructions per wavefront and tile
    constexpr int D = S - 1;                      // tiles in flight ahead
    constexpr int BT = KS >= 32 ? 4 : 8;          // LDS reads issued a batch ahead of the MFMAs
    static_assert(U >= 16 && IPW >= 1 && IPW * 1024 * kRgWaves == SLOT, "tile shape");
    static_assert(S >= 2 && (S & (S - 1)) == 0 && KS % BT == 0, "ring size");
    __shared__ __attribute__((aligned(16))) unsigned char ring[S * SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char stage_all[kRgWaves * kRwStage];
    __shared__ float bias_s[kRgWaves * 32];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int64_t G = gridDim.x;
    const int64_t t0 = blockIdx.x;
    if (t0 >= n_tiles) return;
    const bool has = wave < NB;                   // wavefront-uniform
    // with PP, of wavefronts w and w + 4 (which share a SIMD) the second
    // finishes tile k - 1 before multiplying tile k, so that its epilogue
    // runs while the first one's MFMAs do, and the other way round (its
    // accumulators then live across the barrier: too many registers at K = 512)
    const bool late = PP && wave >= kRgWaves / 2;
    unsigned char* stage = stage_all + wave * kRwStage;

    for (int n = tid; n < kRgWaves * 32; n += kRgWaves * 64) bias_s[n] = bias && n < N ? bias[n] : 0.f;
    uint4 w[KS];
    {
        const T* col = Bp + static_cast<int64_t>(wave * 32 + l32) * Kt + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            w[ks] = has ? *reinterpret_cast<const uint4*>(col + ks * 16) : make_uint4(0, 0, 0, 0);
    }
    // the weights and the bias are in before any direct load is counted
    wait_vm_lgkm0<0>();
    __syncthreads();

    // sources of this thread's direct loads: instruction m writes bytes
    // [1024 j, 1024 j + 1024) of a slot, j = wave * IPW + m.  Per m, two
    // registers: the column in its operand (-1: a unit that reads as zero)
    // and a packed word: the row in the tile (bits 0-4), the operand (bit 5:
    // A2) and the elements inside the operand of a partly covered unit
    // (bits 8-11; 8 when the unit is whole)
    int scol[IPW], sinf[IPW];
#pragma unroll
    for (int m = 0; m < IPW; ++m) {
        const int q = (wave * IPW + m) * 64 + lane;
        const int r = q / U, p = q % U;
        const int64_t k0 = static_cast<int64_t>(p ^ (r & 15)) * 8;
        int col = -1, second = 0, n = 8;
        if (A.a1 && k0 < A.k1p) {
            if (k0 < A.k1) {
                col = static_cast<int>(k0);
                if (A.k1 - k0 < 8) n = static_cast<int>(A.k1 - k0);
            }
        } else if (A.a2 && k0 < A.k1p + A.k2p) {
            if (k0 - A.k1p < A.k2) {
                col = static_cast<int>(k0 - A.k1p);
                second = 1;
                if (A.k2 - (k0 - A.k1p) < 8) n = static_cast<int>(A.k2 - (k0 - A.k1p));
            }
        }
        scol[m] = col;
        sinf[m] = r | (second << 5) | (n << 8);
    }
    const int wbase = wave * IPW * 1024;
    const uint32_t ring_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)ring));
    auto slot_of = [](int64_t k) { return static_cast<int>(k & (S - 1)) * SLOT; };
    auto dma = [&](int64_t k, int64_t tile) __attribute__((always_inline)) {
        const uint32_t dst = ring_lds + static_cast<uint32_t>(slot_of(k) + wbase);
#pragma unroll
        for (int m = 0; m < IPW; ++m) {
            const int64_t row = tile * kRgRows + (sinf[m] & 31);
            const bool second = sinf[m] & 32;
            const T* base = second ? A.a2 : A.a1;
            const int64_t ld = second ? A.lda2 : A.lda1;
            const int64_t lim = second ? A.M : A.m1;
            const void* g = scol[m] >= 0 && row < lim ? static_cast<const void*>(base + row * ld + scol[m])
                                                      : static_cast<const void*>(&g_ring_zero);
            lds_direct_load16(g, dst + m * 1024);
        }
    };
    auto sink_stores = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < kRgStores; ++i) g_ring_sink[wave * 64 + lane] = make_uint4(0, 0, 0, 0);
    };
    // wait for this thread's loads of tile k + 1 (the count is explained
    // below), zero the part past the operand of the partly covered units
    // among them, and meet the workgroup
    auto arrive = [&](int64_t k_next) __attribute__((always_inline)) {
        constexpr int kAfterHas = (D - 1) * IPW + D * kRgStores;
        constexpr int kAfterIdle = (D - 1) * IPW;
        mem_order();
        if (has) wait_vm_lgkm0<kAfterHas>();
        else wait_vm_lgkm0<kAfterIdle>();
        mem_order();
        if (fixup) {
            unsigned char* base = ring + slot_of(k_next) + wbase + lane * 16;
#pragma unroll
            for (int m = 0; m < IPW; ++m) {
                const int n = sinf[m] >> 8;
                if (n < 8) {
                    uint4* u = reinterpret_cast<uint4*>(base + m * 1024);
                    *u = keep_first<T>(*u, n);
                }
            }
            mem_order();
            wait_lgkm0();
        }
        mem_order();
        __builtin_amdgcn_s_barrier();
        mem_order();
    };

    // byte offset in a slot of row l32's unit 2 i + h (i < 8) after the
    // permutation; unit 16 b + c lies 256 b bytes further
    int off8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) off8[i] = l32 * ROWB + (((2 * i + h) ^ (l32 & 15)) << 4);

    f32x16_t acc;
    auto multiply = [&](int64_t k) __attribute__((always_inline)) {
        const unsigned char* rp = ring + slot_of(k);
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        uint4 ab[2][BT];
        auto rd = [&](auto b_c, uint4 (&dst)[BT]) __attribute__((always_inline)) {
            constexpr int b = decltype(b_c)::value;
#pragma unroll
            for (int i = 0; i < BT; ++i) {
                const int ks = b * BT + i;
                dst[i] = *reinterpret_cast<const uint4*>(rp + off8[ks & 7] + 256 * (ks >> 3));
            }
        };
        rd(std::integral_constant<int, 0>{}, ab[0]);
        static_for<0, KS / BT>([&](auto b_c) __attribute__((always_inline)) {
            constexpr int b = decltype(b_c)::value;
            if constexpr (b + 1 < KS / BT) rd(std::integral_constant<int, b + 1>{}, ab[(b + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < BT; ++i)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w[b * BT + i]),
                                                             __builtin_bit_cast(bf16x8_t, ab[b & 1][i]), acc, 0, 0,
                                                             0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    // bias, one rounding, staged as row l32, columns 8q + 4h .. +3 of the
    // block, then stored as 16-byte row pieces (N is a multiple of 8)
    auto finish = [&](int64_t tile) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 bv = *reinterpret_cast<const float4*>(bias_s + wave * 32 + 8 * q + 4 * h);
            const float y[4] = {acc[4 * q] + bv.x, acc[4 * q + 1] + bv.y, acc[4 * q + 2] + bv.z,
                                acc[4 * q + 3] + bv.w};
            *reinterpret_cast<uint2*>(stage + l32 * 80 + (8 * q + 4 * h) * 2) =
                make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < kRgStores; ++i) {
            const int r = (lane >> 2) + 16 * i, c = lane & 3;
            const int64_t grow = tile * kRgRows + r;
            const int64_t col = static_cast<int64_t>(wave) * 32 + c * 8;
            const bool inside = grow < A.M && col < N;
            uint4 v = *reinterpret_cast<const uint4*>(stage + r * 80 + c * 16);
#pragma unroll
            for (int pass = 0; pass < 2; ++pass) {
                T* dst;
                if (pass == 0) {
                    if (!e.pre) continue;
                    dst = e.pre;
                } else {
                    dst = e.c;
                    if (e.relu) v = relu_bf16x8(v);
                }
                uint4* p = inside ? reinterpret_cast<uint4*>(dst + grow * e.ldc + col) : &g_ring_sink[wave * 64 + lane];
                *p = v;
            }
        }
        __builtin_amdgcn_wave_barrier();
    };

    // Vector-memory operations issued after tile k + 1's direct loads when
    // step k waits for them: the stores of the step that issued them, then
    // D - 1 more steps of loads and stores (each step issues at least
    // kRgStores stores per wavefront with a block, and the prologue issues
    // sink stores in place of the steps before the first, so the count
    // holds there too).
    const int64_t steps = (n_tiles - t0 + G - 1) / G;
    for (int v = 0; v < D; ++v) {
        dma(v, t0 + v * G);
        mem_order();
        if (has) sink_stores();
        mem_order();
    }
    arrive(0);
    for (int64_t k = 0; k < steps; ++k) {
        // slot (k + D) % S was multiplied in the step before and every
        // wavefront has passed the barrier since
        dma(k + D, t0 + (k + D) * G);
        mem_order();
        if (has) {
            if (late) {
                if (k > 0) finish(t0 + (k - 1) * G);
                else sink_stores();
                mem_order();
                multiply(k);
            } else {
                multiply(k);
                mem_order();
                finish(t0 + k * G);
            }
        }
        arrive(k + 1);
    }
    if (has && late) finish(t0 + (steps - 1) * G);
    // no direct load may still be writing LDS when the workgroup ends
    wait_vm_lgkm0<0>();
}

template <int KS, int S, bool PP, int WPE>
sag_status launch_nn_ring(const AOperand<uint16_t>& ao, const uint16_t* B, int64_t Kt, int64_t N,
                          const EpiT<uint16_t>& e, const float* bias, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(&gemm_nn_ring<KS, S, PP, WPE>);
    // The wait counts assume that no vector-memory load of the compiler's own
    // runs in the loop; register spills would add scratch loads whose waits
    // the compiler counts without the direct loads it cannot see.  An
    // instance with a private segment is therefore never launched.
    static const bool spill_free = [fn] {
        hipFuncAttributes a{};
        return hipFuncGetAttributes(&a, fn) == hipSuccess && a.localSizeBytes == 0;
    }();
    if (!spill_free) return SAG_E_UNSUPPORTED;
    const int NB = static_cast<int>(cdiv(N, 32));
    // persistent workgroups: exactly as many as are resident at once
    static const int per_cu = [fn] {
        int nb = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kRgWaves * 64, 0) == hipSuccess && nb > 0 ? nb
                                                                                                                : 1;
    }();
    const int64_t n_tiles = cdiv(ao.M, kRgRows);
    int64_t grid = static_cast<int64_t>(device_cus()) * per_cu;
    if (grid > n_tiles) grid = n_tiles;
    const int fixup = (ao.a1 && ao.k1 % 8) || (ao.a2 && ao.k2 % 8);
    gemm_nn_ring<KS, S, PP, WPE><<<dim3(static_cast<unsigned>(grid)), kRgWaves * 64, 0, s>>>(ao, B, Kt, N, NB,
                                                                                            n_tiles, e, bias, fixup);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

#ifndef SAG_NN_RING
#define SAG_NN_RING 1
#endif

// The ring kernel for bf16 without a mask or an addend, 128 < N <= 256 with
// N a multiple of 8 (one 32-column block per wavefront, whole 16-byte
// stores) and a packed K of 256 or 512; SAG_E_UNSUPPORTED otherwise.  (At
// K = 128 the register-prefetch kernel runs two workgroups per CU and is
// faster: 0.40 against 0.44 ms for 2.45M rows to 256 columns.)
sag_status try_nn_ring(const AOperand<uint16_t>& ao, const uint16_t* B, int64_t Kt, int64_t N,
                       const EpiT<uint16_t>& e, const float* bias, hipStream_t s) {
    if (!SAG_NN_RING || e.add || ao.mask || N % 8) return SAG_E_UNSUPPORTED;
    const int64_t NB = cdiv(N, 32);
    if (NB <= 4 || NB > kRgWaves) return SAG_E_UNSUPPORTED;
    switch (Kt) {
        case 256: return launch_nn_ring<16, 8, true, 1>(ao, B, Kt, N, e, bias, s);
        case 512: return launch_nn_ring<32, 4, false, 1>(ao, B, Kt, N, e, bias, s);
        default: return SAG_E_UNSUPPORTED;
    }
}

// ---- TN (weight gradient) -----------------------------------------------------------
// C[k, n] = sum over a chunk of rows m of A[m, k] B[m, n].  Tile: KT rows of C
// (K up to 512 in one tile) by BNT columns; 8 wavefronts, WK along K by WN
// along N, each owning a 64 x TNW block of C.  Steps of 32 rows of A and B
// are copied row-major into padded LDS tiles by whole-line loads (two steps
// in flight in registers, one barrier per step); the MFMA reduction runs
// over m, so bf16 operands are read with the LDS transpose load: for four
// consecutive rows and sixteen columns, lane i of a 16-lane group receives
// column i of the four rows.  Two such reads give a lane the eight m values
// of its column that one 32x32x16 MFMA takes.  fp32 operands (one m per
// lane half) are plain reads.  The column sums of B (the bias gradient) are
// kept in the registers that load B.  The tiles of one row chunk run on the
// same XCD, so the rows they share are read from HBM once.
constexpr int kTnThreads = 512;
constexpr int kTnRows = 32;                       // rows per step

typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <class T> constexpr int tn_pad() { return sizeof(T) == 2 ? 64 : 128; }   // bytes after each LDS row
template <class T, int KT, int BNT> constexpr int tn_stage_bytes() {
    return kTnRows * (KT * static_cast<int>(sizeof(T)) + tn_pad<T>()) +
           kTnRows * (BNT * static_cast<int>(sizeof(T)) + tn_pad<T>());
}

template <class T, int KT, int BNT, bool MASK>
__global__ __launch_bounds__(kTnThreads, 1) void gemm_tn(AOperand<T> A, const T* __restrict__ B, int64_t ldb,
                                                         const T* __restrict__ mask, int64_t ldmask, int64_t N,
                                                         int64_t n_ktile, int64_t n_ntile, int64_t rows_per_chunk,
                                                         float* __restrict__ part, int64_t ldp_k, int64_t ldp_n,
                                                         float* __restrict__ part_cs) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int ES = static_cast<int>(sizeof(T));
    constexpr int V = Vec<T>::N;
    constexpr int PA = KT * ES + tn_pad<T>(), PB = BNT * ES + tn_pad<T>();    // LDS row pitches
    constexpr int SA = kTnRows * PA;
    constexpr int STAGE = tn_stage_bytes<T, KT, BNT>();
    constexpr int WK = KT / 64, WN = 8 / WK;
    constexpr int TNW = BNT / WN;                     // wave tile: 64 x TNW
    constexpr int NBK = 2, NBN = TNW / 32;
    static_assert(TNW >= 32 && TNW % 32 == 0, "wave tile too narrow");
    constexpr int UPA = KT / V, UPB = BNT / V;        // 16-byte units per row
    constexpr int NA = kTnRows * UPA, NBU = kTnRows * UPB;
    constexpr int UA = (NA + kTnThreads - 1) / kTnThreads, UB = (NBU + kTnThreads - 1) / kTnThreads;

    const int64_t tiles = n_ktile * n_ntile;
    const int64_t logical = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t chunk = logical / tiles, tt = logical % tiles;
    const int64_t k0 = (tt / n_ntile) * KT;
    const int64_t n0 = (tt % n_ntile) * BNT;
    const int64_t m_begin = chunk * rows_per_chunk;
    const int64_t m_end = min(A.M, m_begin + rows_per_chunk);
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wk = wave % WK, wn = wave / WK;
    const bool do_cs = part_cs && k0 == 0;
    const int64_t lastn = (N + V - 1) / V * V - V;    // last 16-byte unit of a B row

    // the A units of this thread keep their column for the whole kernel:
    // source pointer at that column, row pitch and the first row that reads
    // as zero (m1 for block 1, M for block 2, 0 past both blocks)
    const T* abase[UA];
    int64_t ald[UA], alim[UA];
#pragma unroll
    for (int j = 0; j < UA; ++j) {
        const int q = t + j * kTnThreads;
        const int64_t kv = k0 + (q % UPA) * V;
        const int64_t last1 = (A.k1 + V - 1) / V * V - V, last2 = (A.k2 + V - 1) / V * V - V;
        if (A.a1 && kv < A.k1p) {
            abase[j] = A.a1 + (kv < last1 ? kv : last1);
            ald[j] = A.lda1;
            alim[j] = A.m1;
        } else if (A.a2 && kv < A.k1p + A.k2p) {
            abase[j] = A.a2 + (kv - A.k1p < last2 ? kv - A.k1p : last2);
            ald[j] = A.lda2;
            alim[j] = A.M;
        } else {
            abase[j] = A.safe;
            ald[j] = 0;
            alim[j] = 0;
        }
    }
    // Every call issues the same loads, whatever the step or the thread: rows
    // are clamped into the operands and units past a step's tile load a
    // clamped row too (they are never written to LDS), so the compiler's
    // wait counts stay exact and a wait for one step never drains the loads
    // of the steps behind it.
    uint4 ra[2][UA], rb[2][UB], rm[2][UB];
    auto load = [&](auto buf_c, int64_t m0) {
        constexpr int bsel = decltype(buf_c)::value;
#pragma unroll
        for (int j = 0; j < UA; ++j) {
            const int q = t + j * kTnThreads;
            const int64_t row = m0 + q / UPA;
            const int64_t rc = row < alim[j] ? row : (alim[j] > 0 ? alim[j] - 1 : 0);
            ra[bsel][j] = *reinterpret_cast<const uint4*>(abase[j] + rc * ald[j]);
        }
#pragma unroll
        for (int j = 0; j < UB; ++j) {
            const int q = t + j * kTnThreads;
            int64_t row = m0 + q / UPB;
            row = row < A.M ? row : A.M - 1;
            int64_t col = n0 + (q % UPB) * V;
            col = col < lastn ? col : lastn;
            rb[bsel][j] = *reinterpret_cast<const uint4*>(B + row * ldb + col);
            if constexpr (MASK) rm[bsel][j] = *reinterpret_cast<const uint4*>(mask + row * ldmask + col);
        }
    };
    float cs[UB][V];
#pragma unroll
    for (int j = 0; j < UB; ++j)
#pragma unroll
        for (int e = 0; e < V; ++e) cs[j][e] = 0.f;
    // masks B, zeroes rows past the chunk, adds B into the column sums and
    // writes the step into stage st
    auto store = [&](auto buf_c, int st, int64_t m0) {
        constexpr int bsel = decltype(buf_c)::value;
        unsigned char* As = lds_raw + st * STAGE;
        unsigned char* Bs = As + SA;
        const bool tail = m0 + kTnRows > m_end;
#pragma unroll
        for (int j = 0; j < UA; ++j) {
            const int q = t + j * kTnThreads;
            if (q < NA) {
                uint4 v = ra[bsel][j];
                const int64_t row = m0 + q / UPA;
                if (row >= m_end || row >= alim[j]) v = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4*>(As + (q / UPA) * PA + (q % UPA) * 16) = v;
            }
        }
#pragma unroll
        for (int j = 0; j < UB; ++j) {
            const int q = t + j * kTnThreads;
            if (q < NBU) {
                uint4 v = rb[bsel][j];
                if constexpr (MASK) v = apply_mask<T>(v, rm[bsel][j]);
                if (tail && m0 + q / UPB >= m_end) v = make_uint4(0, 0, 0, 0);
                if (do_cs) {
                    float f[V];
                    unpack<T>(v, f);
#pragma unroll
                    for (int e = 0; e < V; ++e) cs[j][e] += f[e];
                }
                *reinterpret_cast<uint4*>(Bs + (q / UPB) * PB + (q % UPB) * 16) = v;
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

    // operand read offsets (bytes within a stage tile)
    const int g = lane >> 4, i16 = lane & 15;
    const int q4 = i16 >> 2, r4 = i16 & 3;
    auto compute = [&](int st) {
        const unsigned char* As = lds_raw + st * STAGE;
        const unsigned char* Bs = As + SA;
        if constexpr (kBf16) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {           // 16 rows per MFMA
                const int mrow = 16 * s + 8 * (g >> 1) + q4;
                bf16x8_t xa[NBK], yb[NBN];
#pragma unroll
                for (int i = 0; i < NBK; ++i) {
                    const int col = wk * 64 + 32 * i + 16 * (g & 1) + 4 * r4;
                    const unsigned char* p = As + mrow * PA + col * 2;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(p));
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(p + 4 * PA));
                    xa[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int j = 0; j < NBN; ++j) {
                    const int col = wn * TNW + 32 * j + 16 * (g & 1) + 4 * r4;
                    const unsigned char* p = Bs + mrow * PB + col * 2;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(p));
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) i16x4_t*)(p + 4 * PB));
                    yb[j] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int i = 0; i < NBK; ++i)
#pragma unroll
                    for (int j = 0; j < NBN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[i], yb[j], acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < kTnRows / 2; ++s) {   // 2 rows per MFMA, one per lane half
                const int mrow = 2 * s + (lane >> 5);
                float xa[NBK], yb[NBN];
#pragma unroll
                for (int i = 0; i < NBK; ++i)
                    xa[i] = *reinterpret_cast<const float*>(As + mrow * PA + (wk * 64 + 32 * i + (lane & 31)) * 4);
#pragma unroll
                for (int j = 0; j < NBN; ++j)
                    yb[j] = *reinterpret_cast<const float*>(Bs + mrow * PB + (wn * TNW + 32 * j + (lane & 31)) * 4);
#pragma unroll
                for (int i = 0; i < NBK; ++i)
#pragma unroll
                    for (int j = 0; j < NBN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(xa[i], yb[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    const int64_t nsteps = m_begin < m_end ? (m_end - m_begin + kTnRows - 1) / kTnRows : 0;
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    load(I0{}, m_begin);
    store(I0{}, 0, m_begin);
    load(I1{}, m_begin + kTnRows);
    load(I0{}, m_begin + 2 * kTnRows);
    __syncthreads();
    // step s: write step s+1 (register buffer (s+1)%2) into stage (s+1)%2,
    // refill that buffer with step s+3, then multiply stage s%2.  Steps run
    // in pairs; past the chunk the stores write zeros and the loads read
    // clamped rows, and only the multiply is skipped (a uniform branch with
    // no memory loads in it).
    for (int64_t s0 = 0; s0 < nsteps; s0 += 2) {
        static_for<0, 2>([&](auto dc) {
            constexpr int d = decltype(dc)::value;
            const int64_t s = s0 + d;
            store(std::integral_constant<int, 1 - d>{}, 1 - d, m_begin + (s + 1) * kTnRows);
            load(std::integral_constant<int, 1 - d>{}, m_begin + (s + 3) * kTnRows);
            if (s < nsteps) compute(d);
            __syncthreads();
        });
    }

    float* out = part + chunk * ldp_k * ldp_n;
#pragma unroll
    for (int i = 0; i < NBK; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j) {
            const int64_t col = n0 + wn * TNW + j * 32 + lane % 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = k0 + wk * 64 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
                out[row * ldp_n + col] = acc[i][j][r];
            }
        }
    if (do_cs) {
        // column sums: the per-thread sums of each step row, added in row order
        float* red = reinterpret_cast<float*>(lds_raw);      // [kTnRows][BNT]
#pragma unroll
        for (int j = 0; j < UB; ++j) {
            const int q = t + j * kTnThreads;
            if (q < NBU)
#pragma unroll
                for (int e = 0; e < V; ++e) red[(q / UPB) * BNT + (q % UPB) * V + e] = cs[j][e];
        }
        __syncthreads();
        if (t < BNT) {
            float sum = 0.f;
            for (int r = 0; r < kTnRows; ++r) sum += red[r * BNT + t];
            part_cs[chunk * ldp_n + n0 + t] = sum;
        }
    }
}

// C[k, n] = sum over chunks of the partials, in chunk order.
// p[0] + p[stride] + ... + p[(n-1) stride], added in that order; eight loads
// are issued before their additions.
__device__ __forceinline__ float sum_chunks(const float* __restrict__ p, int64_t stride, int64_t n) {
    float s = 0.f;
    int64_t c = 0;
    for (; c + 8 <= n; c += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p[(c + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; c < n; ++c) s += p[c * stride];
    return s;
}

__global__ void tn_reduce(const float* __restrict__ part, int64_t n_chunks, int64_t ldp_k, int64_t ldp_n,
                          int64_t k1, int64_t k1p, int64_t k2, int64_t N, float* __restrict__ C, int64_t ldc,
                          const float* __restrict__ part_cs, float* __restrict__ colsum) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t rows = k1 + k2;
    if (idx < rows * N) {
        const int64_t k = idx / N, n = idx % N;
        const int64_t kv = k < k1 ? k : k1p + (k - k1);
        C[k * ldc + n] = sum_chunks(part + kv * ldp_n + n, ldp_k * ldp_n, n_chunks);
    }
    if (colsum && idx < N) colsum[idx] = sum_chunks(part_cs + idx, ldp_n, n_chunks);
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

// Device properties, queried once per process (thread-safe static
// initialisation): the library assumes the devices a process uses are alike.
size_t max_lds_per_block() {
    static const size_t lds = [] {
        int dev = 0, v = 0;
        return hipGetDevice(&dev) == hipSuccess &&
                       hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0
                   ? static_cast<size_t>(v)
                   : static_cast<size_t>(65536);
    }();
    return lds;
}

template <class T, int BN, bool MASK, int PD>
sag_status launch_nn(const AOperand<T>& ao, const T* B, int64_t Kt, int64_t N, const EpiT<T>& e,
                     const float* bias, hipStream_t s) {
    const size_t lds = static_cast<size_t>(BN) * Kt * sizeof(T) + static_cast<size_t>(kNnWaves) * kNnTile;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_nn<T, BN, MASK, PD>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(max_lds_per_block()));
    SAG_CHECK_HIP(attr);
    const int64_t n_nblk = cdiv(N, BN);
    const int64_t n_blk = cdiv(ao.M, kNnRows);
    int64_t n_mgroups = device_cus() / n_nblk;
    if (n_mgroups < 1) n_mgroups = 1;
    const int64_t need = cdiv(n_blk, kNnWaves);
    if (n_mgroups > need) n_mgroups = need;
    gemm_nn<T, BN, MASK, PD><<<dim3(static_cast<unsigned>(n_nblk * n_mgroups)), kNnWaves * 64, lds, s>>>(
        ao, B, Kt, N, n_nblk, n_mgroups, n_blk, e, bias);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

// Chunks in flight: four where the registers allow (no mask; fp32 only
// below 128 columns), else two.
template <class T, int BN>
sag_status launch_nn_bn(const AOperand<T>& ao, const T* B, int64_t Kt, int64_t N, const EpiT<T>& e,
                        const float* bias, hipStream_t s) {
    const bool pd4 = (Kt / (128 / static_cast<int64_t>(sizeof(T)))) % 4 == 0;
    if (ao.mask) {
        if constexpr (sizeof(T) == 4 && BN == 128)
            return fail(SAG_E_UNSUPPORTED, "gemm: no fp32 masked kernel for 128 columns");
        else
            return launch_nn<T, BN, true, 2>(ao, B, Kt, N, e, bias, s);
    }
    if constexpr (sizeof(T) == 4 && BN == 128) return launch_nn<T, BN, false, 2>(ao, B, Kt, N, e, bias, s);
    else
        return pd4 ? launch_nn<T, BN, false, 4>(ao, B, Kt, N, e, bias, s)
                   : launch_nn<T, BN, false, 2>(ao, B, Kt, N, e, bias, s);
}

// LDS bytes the NN kernel needs for a column block of bn over Kt.
inline size_t nn_lds_bytes(int64_t bn, int64_t Kt, sag_dtype dt) {
    return static_cast<size_t>(bn) * Kt * elt_size(dt) + static_cast<size_t>(kNnWaves) * kNnTile;
}

#ifndef SAG_NN_RW
#define SAG_NN_RW 1
#endif
int g_nn_rw = SAG_NN_RW;
bool nn_rw_enabled() { return g_nn_rw != 0; }

template <class T>
sag_status nn_typed(int64_t M, int64_t N, const GemmA& A, const void* Bp, sag_dtype dt, void* C, int64_t ldc,
                    const Epilogue& epi, hipStream_t s) {
    AOperand<T> ao = make_aop<T>(A, M, dt, Bp, kchunk(dt));
    const int64_t Kt = k_total(A.a1 ? A.k1 : 0, A.a2 ? A.k2 : 0, dt);
    EpiT<T> e{static_cast<T*>(C), ldc, static_cast<T*>(epi.pre), static_cast<const T*>(epi.addend),
              epi.ld_add, epi.addend ? epi.n_add : 0, epi.bias, epi.relu};
    const T* B = static_cast<const T*>(Bp);
    if constexpr (sizeof(T) == 2) {
        if (nn_rw_enabled()) {
            sag_status st = try_nn_ring(ao, B, Kt, N, e, epi.bias, s);
            if (st != SAG_E_UNSUPPORTED) return st;
            st = try_nn_rw(ao, B, Kt, N, e, epi.bias, s);
            if (st != SAG_E_UNSUPPORTED) return st;
        }
    }
    // widest column block whose slice of B fits in LDS beside the tiles
    const size_t lds = max_lds_per_block();
    const int64_t n32 = round_up(N, 32);
    // (fp32 with a mask stays at 64 columns: 128 would spill registers)
    const bool w128 = !(sizeof(T) == 4 && ao.mask);
    if (w128 && n32 >= 128 && nn_lds_bytes(128, Kt, dt) <= lds)
        return launch_nn_bn<T, 128>(ao, B, Kt, N, e, epi.bias, s);
    if (n32 >= 64 && nn_lds_bytes(64, Kt, dt) <= lds) return launch_nn_bn<T, 64>(ao, B, Kt, N, e, epi.bias, s);
    if (nn_lds_bytes(32, Kt, dt) <= lds) return launch_nn_bn<T, 32>(ao, B, Kt, N, e, epi.bias, s);
    return fail(SAG_E_UNSUPPORTED, "gemm: K too large for one LDS-resident slice of B");
}

struct TnPlan {
    int kt, bnt;
    int64_t n_ktile, n_ntile, n_chunks, rows_per_chunk, ldp_k, ldp_n;
};

// The chunk count depends on M and N only, so workspace sizes grow with K.
TnPlan tn_plan(int64_t M, int64_t Kv, int64_t N, sag_dtype dt) {
    TnPlan p;
    const int64_t kv = Kv > 0 ? Kv : 1;
    // (fp32 stops at 256: a 512 tile and its B slice would not fit twice in LDS)
    p.kt = kv <= 128 ? 128 : ((kv <= 256 || dt != SAG_BF16) ? 256 : 512);
    p.bnt = (N <= 64 && p.kt != 128) ? 64 : 128;
    p.n_ktile = cdiv(kv, p.kt);
    p.n_ntile = cdiv(N > 0 ? N : 1, p.bnt);
    const int64_t ms = kTnRows;
    const int64_t m = M > 0 ? M : 1;
    int64_t want = cdiv(256, p.n_ntile);
    const int64_t max_chunks = cdiv(m, ms);
    if (want > max_chunks) want = max_chunks;
    p.rows_per_chunk = round_up(cdiv(m, want), ms);
    p.n_chunks = cdiv(m, p.rows_per_chunk);
    p.ldp_k = p.n_ktile * p.kt;
    p.ldp_n = p.n_ntile * p.bnt;
    return p;
}

template <class T, int KT, int BNT, bool MASK>
void launch_tn_m(const TnPlan& p, const AOperand<T>& ao, const void* B, int64_t ldb, const void* mask,
                 int64_t ldmask, int64_t N, float* part, float* pcs, hipStream_t s) {
    constexpr size_t lds = 2 * static_cast<size_t>(tn_stage_bytes<T, KT, BNT>());
    static_assert(lds >= static_cast<size_t>(kTnRows) * BNT * 4, "column-sum buffer");
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_tn<T, KT, BNT, MASK>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(lds));
    (void)attr;
    const unsigned grid = static_cast<unsigned>(p.n_chunks * p.n_ktile * p.n_ntile);
    gemm_tn<T, KT, BNT, MASK><<<grid, kTnThreads, lds, s>>>(
        ao, static_cast<const T*>(B), ldb, static_cast<const T*>(mask), ldmask, N, p.n_ktile, p.n_ntile,
        p.rows_per_chunk, part, p.ldp_k, p.ldp_n, pcs);
}

template <class T, int KT, int BNT>
void launch_tn(const TnPlan& p, const AOperand<T>& ao, const void* B, int64_t ldb, const void* mask, int64_t ldmask,
               int64_t N, float* part, float* pcs, hipStream_t s) {
    if (mask) launch_tn_m<T, KT, BNT, true>(p, ao, B, ldb, mask, ldmask, N, part, pcs, s);
    else launch_tn_m<T, KT, BNT, false>(p, ao, B, ldb, mask, ldmask, N, part, pcs, s);
}

template <class T>
sag_status tn_typed(int64_t M, int64_t N, const GemmA& A, const void* B, int64_t ldb, const void* mask,
                    int64_t ldmask, float* C, int64_t ldc, float* colsum, sag_dtype dt, void* ws, size_t ws_bytes,
                    hipStream_t s) {
    AOperand<T> ao = make_aop<T>(A, M, dt, B, vec_elems(dt));
    const int64_t k1 = ao.k1;
    const int64_t k2 = ao.k2;
    const int64_t Kv = kp(k1, dt) + kp(k2, dt);
    TnPlan p = tn_plan(M, Kv, N, dt);
    Carver c(ws, ws_bytes);
    float* part = c.take<float>(p.n_chunks * p.ldp_k * p.ldp_n);
    float* pcs = c.take<float>(p.n_chunks * p.ldp_n);
    if (!c.fits()) return fail(SAG_E_WORKSPACE, "gemm_tn: workspace too small");
    float* cs = colsum ? pcs : nullptr;
    const int64_t total = (k1 + k2) * N;
    const int64_t work = total > N ? total : N;
    if (M == 0) {
        // a sum over no rows: the reduce over zero chunks writes the zeros
        // into all K1 + K2 rows the caller named (an operand with no rows may
        // come without a pointer), and the product kernel, whose row clamps
        // assume at least one row, does not run
        const int64_t zk1 = C ? A.k1 : 0, zk2 = C ? A.k2 : 0;
        const int64_t zwork = (zk1 + zk2) * N > N ? (zk1 + zk2) * N : N;
        tn_reduce<<<dim3(static_cast<unsigned>(cdiv(zwork, 256))), 256, 0, s>>>(
            part, 0, p.ldp_k, p.ldp_n, zk1, zk1, zk2, N, C, ldc, pcs, colsum);
        SAG_LAUNCH_CHECK();
        return SAG_OK;
    }
    if (p.kt == 512) {
        // (bf16 only: the plan keeps fp32 tiles at 256)
        if constexpr (sizeof(T) == 2) {
            if (p.bnt == 64) launch_tn<T, 512, 64>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
            else launch_tn<T, 512, 128>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
        }
    } else if (p.kt == 256 && p.bnt == 64) launch_tn<T, 256, 64>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    else if (p.kt == 256) launch_tn<T, 256, 128>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    else launch_tn<T, 128, 128>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    SAG_LAUNCH_CHECK();
    tn_reduce<<<dim3(static_cast<unsigned>(cdiv(work, 256))), 256, 0, s>>>(
        part, p.n_chunks, p.ldp_k, p.ldp_n, k1, kp(k1, dt), k2, N, C, ldc, pcs, colsum);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

}  // namespace

bool nn_k_fits(int64_t k1, int64_t k2, sag_dtype dt) {
    return nn_lds_bytes(32, k_total(k1, k2, dt), dt) <= max_lds_per_block();
}

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
        pack_kernel<uint16_t><<<grid, 256, 0, s>>>(src, k1, kpc(k1, dt), k2, Kt, nl, n_pad, static_cast<uint16_t*>(Bp));
    else
        pack_kernel<float><<<grid, 256, 0, s>>>(src, k1, kpc(k1, dt), k2, Kt, nl, n_pad, static_cast<float*>(Bp));
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
    // two K blocks pad K by less than two chunks
    return packed_b_bytes(K + 2 * kchunk(dt), 0, N, dt);
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
