/* Test driver for the oracle's C product under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by test_oracle_sanitized.py).
 *
 * Reads one case from a binary file: int64 n_rows, n_cols, nnz, d, ldx,
 * has_val, n_sel; then indptr[n_rows + 1] (int64), indices[nnz] (int32),
 * val[nnz] (float, when has_val), X[n_cols * ldx] (double), rows[n_sel]
 * (int64).  Writes, as doubles: the full product [n_rows * d], its absolute
 * form, the selected rows [n_sel * d], and the fp32 instantiation
 * [n_rows * d].  Every buffer is allocated to its exact size, so a read or
 * write past any of them is reported by the sanitizer. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_spmm_f64(int64_t n_rows, const int64_t* indptr, const int32_t* indices, const float* val,
                  const double* X, int64_t ldx, int64_t d, double* Y, int64_t ldy, int abs_mode);
void orc_spmm_rows_f64(int64_t n_sel, const int64_t* rows, const int64_t* indptr, const int32_t* indices,
                       const float* val, const double* X, int64_t ldx, int64_t d, double* Y, int64_t ldy,
                       int abs_mode);
void orc_spmm_f32(int64_t n_rows, const int64_t* indptr, const int32_t* indices, const float* val,
                  const float* X, int64_t ldx, int64_t d, float* Y, int64_t ldy, int abs_mode);

static void* take(FILE* f, size_t n, size_t es) {
    void* p = malloc(n * es > 0 ? n * es : 1);
    if (!p || fread(p, es, n, f) != n) {
        fprintf(stderr, "short read\n");
        exit(2);
    }
    return p;
}

static void put(FILE* f, const double* p, size_t n) {
    if (fwrite(p, sizeof(double), n, f) != n) exit(3);
}

int main(int argc, char** argv) {
    if (argc != 3) return 1;
    FILE* in = fopen(argv[1], "rb");
    if (!in) return 1;
    int64_t h[7];
    if (fread(h, sizeof(int64_t), 7, in) != 7) return 2;
    const int64_t n_rows = h[0], n_cols = h[1], nnz = h[2], d = h[3], ldx = h[4], has_val = h[5], n_sel = h[6];
    int64_t* indptr = take(in, (size_t)(n_rows + 1), sizeof(int64_t));
    int32_t* indices = take(in, (size_t)nnz, sizeof(int32_t));
    float* val = has_val ? take(in, (size_t)nnz, sizeof(float)) : NULL;
    double* X = take(in, (size_t)(n_cols * ldx), sizeof(double));
    int64_t* rows = take(in, (size_t)n_sel, sizeof(int64_t));
    fclose(in);

    const size_t ny = (size_t)(n_rows * d), ns = (size_t)(n_sel * d);
    double* Y = malloc(ny ? ny * sizeof(double) : 1);
    double* Ya = malloc(ny ? ny * sizeof(double) : 1);
    double* Ys = malloc(ns ? ns * sizeof(double) : 1);
    float* Xf = malloc(n_cols * ldx ? (size_t)(n_cols * ldx) * sizeof(float) : 1);
    float* Yf = malloc(ny ? ny * sizeof(float) : 1);
    double* Yfd = malloc(ny ? ny * sizeof(double) : 1);
    for (int64_t i = 0; i < n_cols * ldx; ++i) Xf[i] = (float)X[i];

    orc_spmm_f64(n_rows, indptr, indices, val, X, ldx, d, Y, d, 0);
    orc_spmm_f64(n_rows, indptr, indices, val, X, ldx, d, Ya, d, 1);
    orc_spmm_rows_f64(n_sel, rows, indptr, indices, val, X, ldx, d, Ys, d, 0);
    orc_spmm_f32(n_rows, indptr, indices, val, Xf, ldx, d, Yf, d, 0);
    for (size_t i = 0; i < ny; ++i) Yfd[i] = (double)Yf[i];

    FILE* out = fopen(argv[2], "wb");
    if (!out) return 1;
    put(out, Y, ny);
    put(out, Ya, ny);
    put(out, Ys, ns);
    put(out, Yfd, ny);
    fclose(out);
    free(indptr);
    free(indices);
    free(val);
    free(X);
    free(rows);
    free(Y);
    free(Ya);
    free(Ys);
    free(Xf);
    free(Yf);
    free(Yfd);
    return 0;
}
