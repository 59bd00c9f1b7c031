/* CPU oracle (test infrastructure only): CSR sparse x dense product in fp64
 * (and the same loops in fp32, used only to time the oracle as a CPU
 * baseline; parity always uses fp64).
 *
 * Y[r, :] = sum over entries p of row r, in ascending p, of val[p] * X[col[p], :]
 *
 * This is the aggregation A^T H of the CAGNET page's forward-propagation
 * equation, computed output row by output row as in that page's 1D
 * block-row algorithm ("Reducing Communication in Graph Neural Network
 * Training", 1D algorithm section).  Each output row is independent, so rows may
 * be spread over threads; within a row the sum runs in entry order with a
 * separate multiply and add (built with -ffp-contract=off).
 *
 * val == NULL means every entry has value 1.  abs_mode != 0 sums
 * |val| * |X| instead (used for error denominators).
 */
#include <stdint.h>
#include <math.h>

void orc_spmm_f64(int64_t n_rows, const int64_t* indptr, const int32_t* indices,
                  const float* val, const double* X, int64_t ldx, int64_t d,
                  double* Y, int64_t ldy, int abs_mode)
{
    #pragma omp parallel for schedule(dynamic, 256)
    for (int64_t r = 0; r < n_rows; ++r) {
        double* y = Y + r * ldy;
        for (int64_t j = 0; j < d; ++j) y[j] = 0.0;
        for (int64_t p = indptr[r]; p < indptr[r + 1]; ++p) {
            double a = val ? (double)val[p] : 1.0;
            const double* x = X + (int64_t)indices[p] * ldx;
            if (abs_mode) {
                a = fabs(a);
                for (int64_t j = 0; j < d; ++j) y[j] += a * fabs(x[j]);
            } else {
                for (int64_t j = 0; j < d; ++j) y[j] += a * x[j];
            }
        }
    }
}

/* The same product for a chosen subset of output rows: Y[i, :] is row
 * rows[i] of the product.  Used when only sampled rows of a large product are
 * compared. */
void orc_spmm_rows_f64(int64_t n_sel, const int64_t* rows, const int64_t* indptr,
                       const int32_t* indices, const float* val, const double* X,
                       int64_t ldx, int64_t d, double* Y, int64_t ldy, int abs_mode)
{
    #pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n_sel; ++i) {
        int64_t r = rows[i];
        double* y = Y + i * ldy;
        for (int64_t j = 0; j < d; ++j) y[j] = 0.0;
        for (int64_t p = indptr[r]; p < indptr[r + 1]; ++p) {
            double a = val ? (double)val[p] : 1.0;
            const double* x = X + (int64_t)indices[p] * ldx;
            if (abs_mode) {
                a = fabs(a);
                for (int64_t j = 0; j < d; ++j) y[j] += a * fabs(x[j]);
            } else {
                for (int64_t j = 0; j < d; ++j) y[j] += a * x[j];
            }
        }
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* The fp32 instantiation of orc_spmm_f64: the same loops with float
 * accumulators (timing only). */
void orc_spmm_f32(int64_t n_rows, const int64_t* indptr, const int32_t* indices,
                  const float* val, const float* X, int64_t ldx, int64_t d,
                  float* Y, int64_t ldy, int abs_mode)
{
    #pragma omp parallel for schedule(dynamic, 256)
    for (int64_t r = 0; r < n_rows; ++r) {
        float* y = Y + r * ldy;
        for (int64_t j = 0; j < d; ++j) y[j] = 0.0f;
        for (int64_t p = indptr[r]; p < indptr[r + 1]; ++p) {
            float a = val ? val[p] : 1.0f;
            const float* x = X + (int64_t)indices[p] * ldx;
            if (abs_mode) {
                a = fabsf(a);
                for (int64_t j = 0; j < d; ++j) y[j] += a * fabsf(x[j]);
            } else {
                for (int64_t j = 0; j < d; ++j) y[j] += a * x[j];
            }
        }
    }
}
