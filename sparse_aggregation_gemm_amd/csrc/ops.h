// Internal launchers shared by the public entry points and the layers.
#pragma once

#include "common.h"

namespace sag {

// Epilogue applied to every output row of an SpMM or GEMM, in fp32 before
// the single rounding to the output type:
//   y = acc (+ addend[row] if row < n_add) (+ bias);  pre = y;
//   out = relu ? max(y, 0) : y.
struct Epilogue {
    const void* addend = nullptr;   // output type, ld ld_add
    int64_t ld_add = 0;
    int64_t n_add = 0;
    const float* bias = nullptr;    // [d]
    int relu = 0;
    void* pre = nullptr;            // output type, same ld as the output; nullable
    int row_mean = 0;               // SpMM: every value of row r is 1/len(r) (the mean
                                    // normalisation): values not read, each row's sum scaled
    const float* part = nullptr;    // SpMM: fp32 partial rows (ld ld_part) of the same product
    int64_t ld_part = 0;            // over the other part of a hub split, added to each row's
                                    // sum before everything else
};

// Leading dimension of the library's own dense buffers: rows wider than 64
// bytes start on a 128-byte cache line and span whole lines, so a gathered
// row touches as few lines as possible; narrower rows are padded to 16 bytes.
inline int64_t ldv(int64_t d, sag_dtype dt) {
    const int64_t e = elt_size(dt), bytes = (d > 0 ? d : 1) * e;
    return (bytes > 64 ? round_up(bytes, 128) : round_up(bytes, 16)) / e;
}
// A product written into one of the library's own buffers computes the
// buffer's whole pitch (the packed weight reads zeros past its columns): its
// rows go out as whole cache lines, with no ragged element stores and no
// partial-line writes.
inline int64_t full_width(int64_t ld) { return ld; }
inline size_t dense_bytes(int64_t rows, int64_t d, sag_dtype dt) {
    return static_cast<size_t>(rows > 0 ? rows : 0) * ldv(d, dt) * elt_size(dt);
}

// ---- SpMM ----------------------------------------------------------------------
// Y[r, :d] = sum_p val[p] X[idx[p], :d]  for every row of A, with the epilogue.
size_t spmm_ws_bytes(const sag_csr& A, int64_t d);
// Long-row partials of a one-pass product over A's own arrays.
size_t spmm_long_ws_bytes(const sag_csr& A, int64_t d);
sag_status spmm_run(const sag_csr& A, const void* X, int64_t ldx, sag_dtype xt, int64_t d, void* Y,
                    int64_t ldy, sag_dtype yt, const Epilogue& epi, void* ws, size_t ws_bytes,
                    hipStream_t s);
sag_status check_csr(const char* name, const sag_csr* A);
// Only the long rows of a scheduled A (nothing without a schedule): row j of
// the long bin's sum goes to Y row j (compact), with no epilogue but the
// row-mean scaling when A is tagged row_mean.
sag_status spmm_long_run(const sag_csr& A, const void* X, int64_t ldx, sag_dtype dt, int64_t d, void* Y,
                         int64_t ldy, void* ws, size_t ws_bytes, hipStream_t s);

// ---- fused aggregate -> transform ------------------------------------------------
// Out = act(Z W + b) (self false) or act([H_ext[:n_rows] | Z] W + b) (self
// true) with Z = A H_ext summed in LDS (Z stored when non-null).
bool agg_transform_fits(int64_t d_in, int64_t d_out, bool self, sag_dtype dt);
size_t agg_transform_ws_bytes(const sag_csr& A, int64_t d_in, int64_t d_out, bool self, sag_dtype dt);
sag_status agg_transform_run(const sag_csr& A, const void* H_ext, int64_t ldh, int64_t d_in, const void* W,
                             const float* b, int64_t d_out, bool self, int relu, sag_dtype dt, void* Y_pre, void* Out,
                             int64_t ldo, void* Z, int64_t ldz, void* ws, size_t ws_bytes, hipStream_t s);
// ---- dense products (MFMA) -------------------------------------------------------
// Operand A of a GEMM: up to two column blocks along K, each [rows, K_i].
// Rows >= m1 of block 1 read as zero (m1 < M lets block 1 cover only the
// first rows).  mask (nullable) multiplies block 1 by 1[mask > 0].
struct GemmA {
    const void* a1 = nullptr;
    int64_t lda1 = 0, k1 = 0, m1 = 0;
    const void* a2 = nullptr;
    int64_t lda2 = 0, k2 = 0;
    const void* mask = nullptr;
    int64_t ldmask = 0;
};

// Source of a packed B operand: element (k, n) of K-block s and N-block t is
// p[s][t][kk * sk + nn * sn] (kk, nn local indices); a null pointer reads 0.
struct PackSrc {
    const void* p[2][2] = {{nullptr, nullptr}, {nullptr, nullptr}};
    int64_t sk[2][2] = {{0, 0}, {0, 0}};
    int64_t sn[2][2] = {{0, 0}, {0, 0}};
};

// Logical N layout of a packed B: columns [0, n0) come from N-block 0,
// [nsplit, nsplit + n1) from N-block 1, the rest are zero.  Total width
// n_total = nsplit + n1 (or n0 when n1 == 0).
struct NLayout {
    int64_t n0 = 0, nsplit = 0, n1 = 0;
    int64_t total() const { return n1 ? nsplit + n1 : n0; }
};

size_t packed_b_bytes(int64_t k1, int64_t k2, int64_t n_total, sag_dtype dt);
// True when an NN product over K blocks (k1, k2) keeps its weight slice in
// LDS (K up to about 1024 fp32 or 2048 bf16 elements).
bool nn_k_fits(int64_t k1, int64_t k2, sag_dtype dt);
sag_status pack_b(const PackSrc& src, int64_t k1, int64_t k2, const NLayout& nl, sag_dtype dt,
                  void* Bp, hipStream_t s);

// C[M, N] = A Bp with the epilogue (C, pre and addend of type dt, ld ldc).
sag_status gemm_run(int64_t M, int64_t N, const GemmA& A, const void* Bp, sag_dtype dt,
                    void* C, int64_t ldc, const Epilogue& epi, hipStream_t s);

// C[K1 + K2, N] (fp32, ld ldc) = A^T Bm, colsum[N] (nullable) = column sums
// of Bm; Bm = B [M, N] (ld ldb) masked by 1[mask > 0] when mask is given.
size_t gemm_tn_ws_bytes(int64_t M, int64_t K, int64_t N, sag_dtype dt);
sag_status gemm_tn_run(int64_t M, int64_t N, const GemmA& A, const void* B, int64_t ldb,
                       const void* mask, int64_t ldmask, float* C, int64_t ldc, float* colsum,
                       sag_dtype dt, void* ws, size_t ws_bytes, hipStream_t s);

// out[M, N] = G * 1[Y > 0] (all of type dt).
sag_status relu_mask_run(int64_t M, int64_t N, const void* G, int64_t ldg, const void* Y,
                         int64_t ldy, void* out, int64_t ldo, sag_dtype dt, hipStream_t s);

}  // namespace sag
