/*
 * tw_oracle.c -- CPU oracle of the ReLU-gated sparse FFN forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark do.  It shares no code,
 * header, table or helper with the HIP kernels.
 *
 * Source of truth: "Sparser, Faster, Lighter Transformer Language Models
 * Review" (the method's review page).  Every function below names the
 * passage it follows.  All arithmetic is plain IEEE double with a fixed,
 * sequential summation order; inputs arrive as doubles that the Python
 * wrapper widened exactly from bfloat16.  Rows are independent, so they are
 * spread over OpenMP threads; that never changes a result.
 *
 * Layouts (row-major throughout):
 *   x     [M][K]        token rows
 *   wg_t  [N][K]        W_g transposed: row j is column j of the gate matrix
 *   wu_t  [N][K]        W_u transposed
 *   wd    [N][K]        W_d, row j is the j-th row of the down projection
 *   z     [M][N]        gate pre-activation x W_g
 *   cnt   [M][N/T]      TwELL count per (token row, column tile)
 *   idx   [M][N/T][C]   TwELL original hidden index (global column j)
 *   val   [M][N/T][C]   TwELL packed value
 *   y     [M][K]        block output
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int tw_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Plain dot product, k ascending, one accumulator.  Both projections of the
 * block ("Sparser, Faster, Lighter ..." section 1-1, the equation for h_u and
 * h_g) are dot products of a token row with a weight column. */
static double dot(const double *a, const double *b, int K)
{
    double s = 0.0;
    for (int k = 0; k < K; ++k)
        s += a[k] * b[k];
    return s;
}

/* ReLU of the gate, section 1-1: negative pre-activations become exactly
 * zero.  A neuron is active iff its gate value is strictly positive, so +0
 * and -0 are inactive. */
static double relu(double v)
{
    return v > 0.0 ? v : 0.0;
}

/* Gate pre-activation z = x W_g (section 1-1 equation, before the ReLU). */
void tw_oracle_gate(const double *x, const double *wg_t, int M, int K, int N, double *z)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m)
        for (int j = 0; j < N; ++j)
            z[(size_t)m * N + j] = dot(x + (size_t)m * K, wg_t + (size_t)j * K, K);
}

/* TwELL packing of a gate matrix and the overflow routing of its rows.
 *
 * Section 3-4 (TwELL: Tile-wise ELLPACK): the N columns are cut into tiles
 * of width T and, for every token row and tile, the non-zero entries of
 * h_g = ReLU(z) are packed locally: packed values (h_v), the original hidden
 * index of each value (h_I) and the per-(row, tile) count (h_nz).
 *
 * Readings where the page is silent: entries are packed in ascending column
 * order; cnt holds the true count even when it exceeds the capacity C; only
 * the first min(cnt, C) slots are filled (unused slots get idx -1, val 0).
 *
 * Section 3-6 (hybrid format) and 4-3 (static capacity): a row whose count
 * exceeds capacity is routed as a whole to a dense backup, recorded in a
 * binary routing vector.  Here flag[m] = 1 iff some tile of row m holds more
 * than C non-zeros; ovf_rows lists the flagged rows in ascending order, at
 * most R_max of them, and *ovf_count receives the true number of flagged
 * rows, which may exceed R_max (the caller then retries with more room).
 */
void tw_oracle_pack(const double *z, int M, int N, int T, int C, int R_max,
                    int32_t *cnt, int32_t *idx, double *val,
                    uint8_t *flag, int32_t *ovf_rows, int32_t *ovf_count)
{
    const int NT = N / T;
#pragma omp parallel for schedule(dynamic, 16)
    for (int m = 0; m < M; ++m) {
        int over = 0;
        for (int t = 0; t < NT; ++t) {
            const size_t tile = (size_t)m * NT + t;
            int n = 0;
            for (int s = 0; s < C; ++s) {
                idx[tile * C + s] = -1;
                val[tile * C + s] = 0.0;
            }
            for (int j = t * T; j < (t + 1) * T; ++j) {
                const double g = relu(z[(size_t)m * N + j]);
                if (g > 0.0) {
                    if (n < C) {
                        idx[tile * C + n] = j;
                        val[tile * C + n] = g;
                    }
                    ++n;
                }
            }
            cnt[tile] = n;
            if (n > C)
                over = 1;
        }
        flag[m] = (uint8_t)over;
    }
    int r = 0;
    for (int m = 0; m < M; ++m) {
        if (flag[m]) {
            if (r < R_max)
                ovf_rows[r] = m;
            ++r;
        }
    }
    *ovf_count = r;
}

/* Dense gated FFN, section 1-1 equation: h_u = x W_u, h_g = ReLU(x W_g),
 * h = h_u (elementwise) h_g, y = h W_d.  The sum over the hidden index j
 * runs in ascending j with a single accumulator per output element. */
static void dense_row(const double *xm, const double *wg_t, const double *wu_t,
                      const double *wd, int K, int N, double *ym)
{
    for (int k = 0; k < K; ++k)
        ym[k] = 0.0;
    for (int j = 0; j < N; ++j) {
        const double g = relu(dot(xm, wg_t + (size_t)j * K, K));
        const double u = dot(xm, wu_t + (size_t)j * K, K);
        const double h = u * g;
        const double *wdj = wd + (size_t)j * K;
        for (int k = 0; k < K; ++k)
            ym[k] += h * wdj[k];
    }
}

void tw_oracle_dense_ffn(const double *x, const double *wg_t, const double *wu_t,
                         const double *wd, int M, int K, int N, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m)
        dense_row(x + (size_t)m * K, wg_t, wu_t, wd, K, N, y + (size_t)m * K);
}

/* Sparse evaluation from a TwELL packing, section 3-5 equation:
 * y_m = sum over active n of (h_g)_{m,n} (x_m W_{u,:,n}) W_{d,n,:}.
 * Only the packed entries are visited (tiles ascending, slots ascending,
 * which is ascending j).  A row with any tile over capacity takes the dense
 * backup path of section 3-6 instead and is recomputed from x. */
void tw_oracle_sparse_ffn(const double *x, const double *wg_t, const double *wu_t,
                          const double *wd, int M, int K, int N, int T, int C,
                          const int32_t *cnt, const int32_t *idx, const double *val,
                          double *y)
{
    const int NT = N / T;
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        const double *xm = x + (size_t)m * K;
        double *ym = y + (size_t)m * K;
        int over = 0;
        for (int t = 0; t < NT; ++t)
            if (cnt[(size_t)m * NT + t] > C)
                over = 1;
        if (over) {
            dense_row(xm, wg_t, wu_t, wd, K, N, ym);
            continue;
        }
        for (int k = 0; k < K; ++k)
            ym[k] = 0.0;
        for (int t = 0; t < NT; ++t) {
            const size_t tile = (size_t)m * NT + t;
            for (int s = 0; s < cnt[tile]; ++s) {
                const int j = idx[tile * C + s];
                const double g = val[tile * C + s];
                const double u = dot(xm, wu_t + (size_t)j * K, K);
                const double h = u * g;
                const double *wdj = wd + (size_t)j * K;
                for (int k = 0; k < K; ++k)
                    ym[k] += h * wdj[k];
            }
        }
    }
}
