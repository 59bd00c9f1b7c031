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
// K blocks of the NN product are padded to whole MFMA k-steps (16 bf16, 8
// fp32), so that every k-step lies inside one block.
inline int64_t kstep(sag_dtype dt) { return dt == SAG_BF16 ? 16 : 8; }
inline int64_t kpn(int64_t k, sag_dtype dt) { return round_up(k, kstep(dt)); }
// K of a packed B: a multiple of 16 MFMA k-steps when that costs at most
// 16 extra k-steps' worth of padding, else of 8 (the NN kernel keeps that
// many A fragments in flight).
inline int64_t k_total(int64_t k1, int64_t k2, sag_dtype dt) {
    const int64_t kv = kpn(k1, dt) + kpn(k2, dt);
    const int64_t step = kstep(dt);
    return kv >= 16 * step ? round_up(kv, 16 * step) : round_up(kv, 8 * step);
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

    __device__ __forceinline__ const uint4* addr(int64_t r, int64_t k0) const {
        const T* p = safe;
        if (r < M) {
            if (k0 < k1p) {
                if (r < m1) p = a1 + r * lda1 + k0;
            } else if (k0 < k1p + k2p) {
                p = a2 + r * lda2 + (k0 - k1p);
            }
        }
        return reinterpret_cast<const uint4*>(p);
    }
    __device__ __forceinline__ const uint4* mask_addr(int64_t r, int64_t k0) const {
        const T* p = safe;
        if (mask && r < M && r < m1 && k0 < k1p) p = mask + r * ldmask + k0;
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
// gradient).  A workgroup keeps its BN columns of the packed B (all of K) in
// LDS for its whole life; each of its wavefronts streams 32-row blocks of A
// straight from memory into MFMA operands with kDepth 16-byte fragments in
// flight, so the only HBM traffic is A once and C once.  Persistent: one
// workgroup per CU walks the 32-row blocks of its N block.
constexpr int kNnWaves = 8;

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <class T> struct StreamMfma;
// The MFMAs compute transposed blocks, C^T = B^T A^T: B supplies the first
// operand and A the second, so lane l accumulates row l%32 of a 32x32 block
// of C and register r holds column 8*(r/4) + 4*(l/32) + r%4 -- four
// consecutive columns per register quad, stored as one vector.
// bf16: one A load holds k0..k0+7 (lanes 0-31) or k0+8..k0+15 (lanes 32-63),
// exactly the operand of one 32x32x16 MFMA.
template <> struct StreamMfma<uint16_t> {
    static constexpr int KSTEP = 16;
    // Bk: the LDS slice of this k-step, [BN][16]; lane reads n = j*32 + l%32
    template <int NB>
    __device__ static __forceinline__ void step(const uint4& a, const uint16_t* Bk, int lane, f32x16_t (&acc)[NB]) {
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
        const uint16_t* bp = Bk + (lane % 32) * 16 + (lane / 32) * 8;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(bp + j * 32 * 16);
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv, av, acc[j], 0, 0, 0);
        }
    }
};
// fp32: one A load holds k0..k0+3 (lanes 0-31) or k0+4..k0+7 (lanes 32-63);
// four 32x32x2 MFMAs pair k0+s with k0+4+s, and B is read with the same
// pairing, so the products sum over k0..k0+7.
template <> struct StreamMfma<float> {
    static constexpr int KSTEP = 8;
    template <int NB>
    __device__ static __forceinline__ void step(const uint4& a, const float* Bk, int lane, f32x16_t (&acc)[NB]) {
        const f32x4_t av = __builtin_bit_cast(f32x4_t, a);
        const float* bp = Bk + (lane % 32) * 8 + (lane / 32) * 4;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const f32x4_t bv = *reinterpret_cast<const f32x4_t*>(bp + j * 32 * 8);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[q], av[q], acc[j], 0, 0, 0);
        }
    }
};

template <class T, int BN, bool MASK, int kDepth>
__global__ __launch_bounds__(kNnWaves * 64) void gemm_nn(AOperand<T> A, const T* __restrict__ Bp, int64_t Kt,
                                                         int64_t N, int64_t n_nblk, int64_t n_mgroups,
                                                         int64_t n_mblk, EpiT<T> e) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    // B slice of this column block as [k-step][BN][KSTEP]: the fragment of
    // column block j of a k-step sits at a fixed offset, an immediate.
    T* Bs = reinterpret_cast<T*>(lds_raw);
    constexpr int V = Vec<T>::N;
    constexpr int NB = BN / 32;
    constexpr int KSTEP = StreamMfma<T>::KSTEP;
    constexpr int KSV = KSTEP / V;                  // vectors per k-step
    const int64_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t nb = tile % n_nblk, mg = tile / n_nblk;
    const int64_t n0 = nb * BN;
    const int64_t kvec = Kt / V;
    for (int64_t q = threadIdx.x; q < BN * kvec; q += kNnWaves * 64) {
        const int64_t r = q / kvec, c = q % kvec;   // column r, vector c
        const int64_t ks = c / KSV, w = c % KSV;
        *reinterpret_cast<uint4*>(Bs + (ks * BN + r) * KSTEP + w * V) =
            *reinterpret_cast<const uint4*>(Bp + (n0 + r) * Kt + c * V);
    }
    // the bias of the block's columns sits after B, so the epilogue never
    // waits on global memory behind the prefetched fragments
    float* bias_lds = reinterpret_cast<float*>(lds_raw + static_cast<size_t>(BN) * Kt * sizeof(T));
    for (int q = threadIdx.x; q < BN; q += kNnWaves * 64)
        bias_lds[q] = (e.bias && n0 + q < N) ? e.bias[n0 + q] : 0.f;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t stride = n_mgroups * kNnWaves;
    int64_t mb = mg * kNnWaves + wave;
    if (mb >= n_mblk) return;
    const int nks = static_cast<int>(Kt / KSTEP);   // a multiple of kDepth
    const int nks1 = static_cast<int>(A.k1p / KSTEP);                // k-steps of block 1
    // the only k-steps whose fragments need zeroing: the ragged end of block 1
    // and everything from the ragged end of block 2 on
    const int fix1 = A.k1 < A.k1p ? static_cast<int>(A.k1 / KSTEP) : -1;
    const int fix2 = static_cast<int>((A.k1p + A.k2) / KSTEP);
    const int koff = (lane / 32) * (KSTEP / 2);
    const int64_t rl = lane % 32;
    // per-lane bases: row of this block (and the next), shifted by the lane's
    // half of the k-step; the k-step offset is a uniform scalar
    auto bases = [&](int64_t blk, const T*& b1, const T*& b2, const T*& bm) {
        const T *p1, *p2;
        A.row_ptrs(blk * 32 + rl, p1, p2);
        b1 = p1 + koff;
        b2 = p2 + koff - A.k1p;   // block 2 addressed with the virtual column
        if constexpr (MASK) {
            const int64_t r = blk * 32 + rl;
            bm = A.mask + (r < A.M ? r : A.M - 1) * A.ldmask + koff;
        }
    };
    // last 16-byte vector of each block inside its rows (a block's k-step
    // padding may reach past the row's leading dimension)
    const int64_t last1 = (A.k1 + V - 1) / V * V - V, last2 = (A.k2 + V - 1) / V * V - V;
    auto frag_ptr = [&](const T* b1, const T* b2, int ks) -> const uint4* {
        const T* p;
        if (ks == fix1 || ks >= fix2) {
            // edge or past the data (the value is zeroed at use): clamp the
            // lane's column into the block's real vectors
            const int64_t col = static_cast<int64_t>(ks) * KSTEP + koff;
            if (col < A.k1p || !A.a2) {
                const int64_t c = col < last1 ? col : last1;
                p = b1 - koff + c;
            } else {
                const int64_t c2 = col - A.k1p;
                p = b2 - koff + A.k1p + (c2 < last2 ? c2 : last2);
            }
        } else {
            p = ks < nks1 ? b1 + ks * KSTEP : b2 + ks * KSTEP;
        }
        return reinterpret_cast<const uint4*>(p);
    };
    auto mask_ptr = [&](const T* bm_, int ks) -> const uint4* {
        const int64_t col = static_cast<int64_t>(ks) * KSTEP + koff;
        const int64_t c = col < last1 ? col : last1;
        return reinterpret_cast<const uint4*>(bm_ - koff + c);
    };
    uint4 buf[kDepth], mbuf[MASK ? kDepth : 1];
    const T *b1, *b2, *bm = nullptr, *c1, *c2, *cm = nullptr;
    bases(mb, b1, b2, bm);
    static_for<0, kDepth>([&](auto dc) {
        constexpr int d = decltype(dc)::value;
        buf[d] = *frag_ptr(b1, b2, d);
        if constexpr (MASK) mbuf[d] = *mask_ptr(bm, d);
    });
    for (;;) {
        f32x16_t acc[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
        const int64_t mb_next = mb + stride;
        bases(mb_next, c1, c2, cm);
        // rows of this block at or past m1 (or M) read block 1 as zero
        const bool zero_rows = mb * 32 + 31 >= A.m1;
        for (int ks0 = 0; ks0 < nks; ks0 += kDepth) {
            static_for<0, kDepth>([&](auto dc) {
                constexpr int d = decltype(dc)::value;
                const int ks = ks0 + d;
                uint4 a = buf[d];
                if constexpr (MASK) {
                    if (ks < nks1) a = apply_mask<T>(a, mbuf[d]);
                }
                if (zero_rows || ks == fix1 || ks >= fix2)
                    a = A.fix(a, mb * 32 + rl, static_cast<int64_t>(ks) * KSTEP + koff);
                int kn = ks + kDepth;
                const T *r1 = b1, *r2 = b2, *rm = bm;
                if (kn >= nks) {
                    kn -= nks;
                    r1 = c1;
                    r2 = c2;
                    rm = cm;
                }
                buf[d] = *frag_ptr(r1, r2, kn);
                if constexpr (MASK) mbuf[d] = *mask_ptr(rm, kn);
                StreamMfma<T>::template step<NB>(a, Bs + static_cast<int64_t>(ks) * BN * KSTEP, lane, acc);
            });
        }
        // epilogue: lane l holds row l%32 of the block; register quad q of
        // column block j holds columns j*32 + 8q + 4(l/32) .. +3
        const int64_t row = mb * 32 + rl;
        if (row < A.M) {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t cl = j * 32 + 8 * q + 4 * (lane / 32);
                    const int64_t col = n0 + cl;
                    if (col >= N) continue;
                    const int n = static_cast<int>(N - col < 4 ? N - col : 4);
                    float y[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) y[t] = acc[j][4 * q + t] + bias_lds[cl + t];
                    if (e.add && row < e.n_add) {
#pragma unroll
                        for (int t = 0; t < 4; ++t)
                            if (t < n) y[t] += to_f32(e.add[row * e.ld_add + col + t]);
                    }
                    if (e.pre) store4<T>(e.pre + row * e.ldc + col, y, n);
                    if (e.relu) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) y[t] = y[t] < 0.f ? 0.f : y[t];
                    }
                    store4<T>(e.c + row * e.ldc + col, y, n);
                }
            }
        }
        mb = mb_next;
        if (mb >= n_mblk) break;
        b1 = c1;
        b2 = c2;
        bm = cm;
    }
}

// ---- TN (weight gradient) -----------------------------------------------------------
// C[k, n] = sum over a chunk of rows m of A[m, k] B[m, n].  Tile: KT rows of C
// (K up to 512 in one tile) by BNT columns; 8 wavefronts, WK along K by WN
// along N.  Each step stages MS rows of A and B in LDS; for bf16 they are
// stored transposed (k-major, m contiguous) because the MFMA reduction runs
// over m, with each thread writing 4 consecutive m values at once.
constexpr int kTnThreads = 512;

template <class T, int KT, int BNT>
__global__ __launch_bounds__(kTnThreads) void gemm_tn(AOperand<T> A, const T* __restrict__ B, int64_t ldb,
                                                      const T* __restrict__ mask, int64_t ldmask, int64_t N,
                                                      int64_t n_ktile, int64_t n_ntile, int64_t rows_per_chunk,
                                                      float* __restrict__ part, int64_t ldp_k, int64_t ldp_n,
                                                      float* __restrict__ part_cs) {
    constexpr bool kBf16 = sizeof(T) == 2;
    constexpr int V = Vec<T>::N;
    constexpr int KI = Mfma<T>::KI;
    constexpr int MS = kBf16 ? 32 : 16;               // rows per step
    constexpr int WK = KT / 64, WN = 8 / WK;
    constexpr int TK = KT / WK, TNW = BNT / WN;       // wave tile
    constexpr int NBK = TK / 32, NBN = TNW / 32;
    static_assert(TNW >= 32 && TNW % 32 == 0, "wave tile too narrow");
    constexpr int LPA = kBf16 ? MS + 8 : KT + 4;
    constexpr int LPB = kBf16 ? MS + 8 : BNT + 4;
    constexpr int SA = kBf16 ? KT * LPA : MS * LPA;
    constexpr int SB = kBf16 ? BNT * LPB : MS * LPB;
    __shared__ __attribute__((aligned(16))) T As[SA];
    __shared__ __attribute__((aligned(16))) T Bs[SB];
    constexpr int ITEMS_A = (MS / 4) * (KT / V);      // 4 rows x one vector each
    constexpr int ITEMS_B = (MS / 4) * (BNT / V);
    static_assert(ITEMS_A <= kTnThreads && ITEMS_B <= kTnThreads, "too many items");

    const int64_t tiles = n_ktile * n_ntile;
    const int64_t chunk = blockIdx.x / tiles;
    const int64_t tt = blockIdx.x % tiles;
    const int64_t k0 = (tt / n_ntile) * KT;
    const int64_t n0 = (tt % n_ntile) * BNT;
    const int64_t m_begin = chunk * rows_per_chunk;
    const int64_t m_end = min(A.M, m_begin + rows_per_chunk);
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    const int wk = wave % WK, wn = wave / WK;
    const bool do_cs = part_cs && k0 == 0;
    // item of this thread: rows 4*rq .. 4*rq+3 of the step, one vector column
    const int a_rq = t % (MS / 4), a_cv = t / (MS / 4);
    const int b_rq = t % (MS / 4), b_cv = t / (MS / 4);

    // raw loads are issued a step ahead; zeroing and masking happen when the
    // step is written to LDS
    uint4 ra[4], rb[4], rm[4];
    int64_t step_m0 = m_begin;
    auto load_step = [&](int64_t m0) {
        if (t < ITEMS_A) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + a_rq * 4 + i;
                ra[i] = *A.addr(row < m_end ? row : A.M, k0 + a_cv * V);
            }
        }
        if (t < ITEMS_B) {
            const int64_t col = n0 + b_cv * V;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = m0 + b_rq * 4 + i;
                const bool ok = row < m_end && col < N;
                rb[i] = *reinterpret_cast<const uint4*>(ok ? B + row * ldb + col : B);
                if (mask) rm[i] = *reinterpret_cast<const uint4*>(ok ? mask + row * ldmask + col : mask);
            }
        }
    };
    auto fix_step = [&]() {
        if (t < ITEMS_A) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = step_m0 + a_rq * 4 + i;
                ra[i] = row < m_end ? A.fix(ra[i], row, k0 + a_cv * V) : make_uint4(0, 0, 0, 0);
            }
        }
        if (t < ITEMS_B) {
            const int64_t col = n0 + b_cv * V;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = step_m0 + b_rq * 4 + i;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (row < m_end && col < N) {
                    v = keep_first<T>(rb[i], static_cast<int>(N - col));
                    if (mask) v = apply_mask<T>(v, rm[i]);
                }
                rb[i] = v;
            }
        }
    };
    auto store_step = [&]() {
        fix_step();
        if constexpr (kBf16) {
            // transpose: element (m, k) goes to As[k][m]; 4 m values per write
            if (t < ITEMS_A) {
                const uint32_t w0[4] = {ra[0].x, ra[0].y, ra[0].z, ra[0].w};
                const uint32_t w1[4] = {ra[1].x, ra[1].y, ra[1].z, ra[1].w};
                const uint32_t w2[4] = {ra[2].x, ra[2].y, ra[2].z, ra[2].w};
                const uint32_t w3[4] = {ra[3].x, ra[3].y, ra[3].z, ra[3].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // halves e of rows m, m+1 (and m+2, m+3) side by side
                    const uint32_t sel_b = (e & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t lo = __builtin_amdgcn_perm(w1[e / 2], w0[e / 2], sel_b);
                    const uint32_t hi = __builtin_amdgcn_perm(w3[e / 2], w2[e / 2], sel_b);
                    *reinterpret_cast<uint2*>(&As[(a_cv * 8 + e) * LPA + a_rq * 4]) = make_uint2(lo, hi);
                }
            }
            if (t < ITEMS_B) {
                const uint32_t w0[4] = {rb[0].x, rb[0].y, rb[0].z, rb[0].w};
                const uint32_t w1[4] = {rb[1].x, rb[1].y, rb[1].z, rb[1].w};
                const uint32_t w2[4] = {rb[2].x, rb[2].y, rb[2].z, rb[2].w};
                const uint32_t w3[4] = {rb[3].x, rb[3].y, rb[3].z, rb[3].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t sel_b = (e & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t lo = __builtin_amdgcn_perm(w1[e / 2], w0[e / 2], sel_b);
                    const uint32_t hi = __builtin_amdgcn_perm(w3[e / 2], w2[e / 2], sel_b);
                    *reinterpret_cast<uint2*>(&Bs[(b_cv * 8 + e) * LPB + b_rq * 4]) = make_uint2(lo, hi);
                }
            }
        } else {
            if (t < ITEMS_A) {
#pragma unroll
                for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&As[(a_rq * 4 + i) * LPA + a_cv * V]) = ra[i];
            }
            if (t < ITEMS_B) {
#pragma unroll
                for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&Bs[(b_rq * 4 + i) * LPB + b_cv * V]) = rb[i];
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
            step_m0 = m0 + MS;
            if (do_cs && t < BNT) {
                if constexpr (kBf16) {
#pragma unroll
                    for (int r = 0; r < MS; ++r) cs += bf16_to_f32(Bs[t * LPB + r]);
                } else {
#pragma unroll
                    for (int r = 0; r < MS; ++r) cs += Bs[r * LPB + t];
                }
            }
#pragma unroll
            for (int ks = 0; ks < MS; ks += KI) {
                typename Mfma<T>::frag fa[NBK], fb[NBN];
                if constexpr (kBf16) {
#pragma unroll
                    for (int i = 0; i < NBK; ++i)
                        fa[i] = Mfma<T>::ld(&As[(wk * TK + i * 32 + lane % 32) * LPA], ks);
#pragma unroll
                    for (int j = 0; j < NBN; ++j)
                        fb[j] = Mfma<T>::ld(&Bs[(wn * TNW + j * 32 + lane % 32) * LPB], ks);
                } else {
                    const int mr = ks + lane / 32;
#pragma unroll
                    for (int i = 0; i < NBK; ++i)
                        fa[i] = reinterpret_cast<const float*>(As)[mr * LPA + wk * TK + i * 32 + lane % 32];
#pragma unroll
                    for (int j = 0; j < NBN; ++j)
                        fb[j] = reinterpret_cast<const float*>(Bs)[mr * LPB + wn * TNW + j * 32 + lane % 32];
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
            const int64_t col = n0 + wn * TNW + j * 32 + lane % 32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = k0 + wk * TK + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + (r % 4);
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

int device_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cus = v;
        else
            cus = 256;
    }
    return cus;
}

size_t max_lds_per_block() {
    static size_t lds = 0;
    if (!lds) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && v > 0)
            lds = static_cast<size_t>(v);
        else
            lds = 65536;
    }
    return lds;
}

template <class T, int BN, bool MASK, int D>
sag_status launch_nn_d(const AOperand<T>& ao, const T* B, int64_t Kt, int64_t N, const EpiT<T>& e, hipStream_t s) {
    const size_t lds = static_cast<size_t>(BN) * Kt * sizeof(T) + BN * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        SAG_CHECK_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_nn<T, BN, MASK, D>),
                                          hipFuncAttributeMaxDynamicSharedMemorySize,
                                          static_cast<int>(max_lds_per_block())));
        attr_set = true;
    }
    const int64_t n_nblk = cdiv(N, BN);
    const int64_t n_mblk = cdiv(ao.M, 32);
    int64_t n_mgroups = device_cus() / n_nblk;
    if (n_mgroups < 1) n_mgroups = 1;
    const int64_t need = cdiv(n_mblk, kNnWaves);
    if (n_mgroups > need) n_mgroups = need;
    gemm_nn<T, BN, MASK, D><<<dim3(static_cast<unsigned>(n_nblk * n_mgroups)), kNnWaves * 64, lds, s>>>(
        ao, B, Kt, N, n_nblk, n_mgroups, n_mblk, e);
    SAG_LAUNCH_CHECK();
    return SAG_OK;
}

template <class T, int BN, bool MASK>
sag_status launch_nn(const AOperand<T>& ao, const T* B, int64_t Kt, int64_t N, const EpiT<T>& e, hipStream_t s) {
    const int64_t nks = Kt / StreamMfma<T>::KSTEP;
    if (nks % 16 == 0) return launch_nn_d<T, BN, MASK, 16>(ao, B, Kt, N, e, s);
    return launch_nn_d<T, BN, MASK, 8>(ao, B, Kt, N, e, s);
}

template <class T>
sag_status nn_typed(int64_t M, int64_t N, const GemmA& A, const void* Bp, sag_dtype dt, void* C, int64_t ldc,
                    const Epilogue& epi, hipStream_t s) {
    AOperand<T> ao = make_aop<T>(A, M, dt, Bp, kstep(dt));
    const int64_t Kt = k_total(A.a1 ? A.k1 : 0, A.a2 ? A.k2 : 0, dt);
    EpiT<T> e{static_cast<T*>(C), ldc, static_cast<T*>(epi.pre), static_cast<const T*>(epi.addend),
              epi.ld_add, epi.addend ? epi.n_add : 0, epi.bias, epi.relu};
    const T* B = static_cast<const T*>(Bp);
    // widest N block whose slice of B fits in LDS
    const size_t lds = max_lds_per_block();
    const int64_t n32 = round_up(N, 32);
    const size_t row = static_cast<size_t>(Kt) * sizeof(T) + sizeof(float);
    // (a 256-column block would need more than the 256 registers a lane has
    // at two wavefronts per SIMD; the column blocks of one row group run on
    // the same XCD, so A is read from HBM about once)
    const bool m = ao.mask != nullptr;
    if (n32 >= 128 && 128 * row <= lds)
        return m ? launch_nn<T, 128, true>(ao, B, Kt, N, e, s) : launch_nn<T, 128, false>(ao, B, Kt, N, e, s);
    if (n32 >= 64 && 64 * row <= lds)
        return m ? launch_nn<T, 64, true>(ao, B, Kt, N, e, s) : launch_nn<T, 64, false>(ao, B, Kt, N, e, s);
    if (32 * row <= lds)
        return m ? launch_nn<T, 32, true>(ao, B, Kt, N, e, s) : launch_nn<T, 32, false>(ao, B, Kt, N, e, s);
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
    p.kt = kv <= 128 ? 128 : (kv <= 256 ? 256 : 512);
    p.bnt = (N <= 64 && p.kt != 128) ? 64 : 128;
    p.n_ktile = cdiv(kv, p.kt);
    p.n_ntile = cdiv(N > 0 ? N : 1, p.bnt);
    const int64_t ms = dt == SAG_BF16 ? 32 : 16;
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

template <class T, int KT, int BNT>
void launch_tn(const TnPlan& p, const AOperand<T>& ao, const void* B, int64_t ldb, const void* mask, int64_t ldmask,
               int64_t N, float* part, float* pcs, hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(p.n_chunks * p.n_ktile * p.n_ntile);
    gemm_tn<T, KT, BNT><<<grid, kTnThreads, 0, s>>>(ao, static_cast<const T*>(B), ldb, static_cast<const T*>(mask),
                                                     ldmask, N, p.n_ktile, p.n_ntile, p.rows_per_chunk, part,
                                                     p.ldp_k, p.ldp_n, pcs);
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
    if (p.kt == 512 && p.bnt == 64) launch_tn<T, 512, 64>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    else if (p.kt == 512) launch_tn<T, 512, 128>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    else if (p.kt == 256 && p.bnt == 64) launch_tn<T, 256, 64>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    else if (p.kt == 256) launch_tn<T, 256, 128>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    else launch_tn<T, 128, 128>(p, ao, B, ldb, mask, ldmask, N, part, cs, s);
    SAG_LAUNCH_CHECK();
    const int64_t total = (k1 + k2) * N;
    const int64_t work = total > N ? total : N;
    tn_reduce<<<dim3(static_cast<unsigned>(cdiv(work, 256))), 256, 0, s>>>(
        part, p.n_chunks, p.ldp_k, p.ldp_n, k1, kp(k1, dt), k2, N, C, ldc, pcs, colsum);
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
        pack_kernel<uint16_t><<<grid, 256, 0, s>>>(src, k1, kpn(k1, dt), k2, Kt, nl, n_pad, static_cast<uint16_t*>(Bp));
    else
        pack_kernel<float><<<grid, 256, 0, s>>>(src, k1, kpn(k1, dt), k2, Kt, nl, n_pad, static_cast<float*>(Bp));
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
