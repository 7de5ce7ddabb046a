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
 * Hybrid storage (training forward), sparse capacity P, backup room R_max:
 *   hy_cnt [M]          non-zeros of each row (the true count)
 *   hy_idx [M][P]       original hidden index of each stored entry
 *   hy_val [M][P]       stored gate value (hy_u, hy_h: up and product values)
 *   route  [M]          1 if the row lives in the dense backup, else 0
 *   bk_rows [R_max]     backup rows in ascending order
 *   bk_g, bk_u, bk_h [R_max][N]  dense gate, up and product rows of the backup
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

/* Hybrid storage of the gate activation, section 3-6 (compact ELL-like rows
 * for most tokens, a dense backup for the few heavy ones, a binary routing
 * vector saying which holds each row) with the static capacities of section
 * 4-3 (at most P stored non-zeros per sparse row, at most R_max backup rows,
 * overflow reported for a retry with more room).  It is built from a TwELL
 * packing, the order of the training pipeline in section 2-2 (TwELL gate,
 * then hybrid storage).
 *
 * Readings where the page is silent: the row's non-zero count is the sum of
 * its TwELL tile counts; a row goes to the backup when that count exceeds P
 * or when one of its tiles exceeded the TwELL capacity C (its packing then
 * lacks entries); a sparse row stores its entries in ascending column order
 * (tiles ascending, slots ascending), the row-wide ELL of section 3-3 with
 * capacity P; unused slots get idx -1, val 0.  hy_cnt is the row's true
 * count for every row.  bk_rows lists the backup rows in ascending order, at
 * most R_max of them, and *bk_count receives their true number. */
void tw_oracle_hybrid_pack(int M, int NT, int C, const int32_t *cnt, const int32_t *idx,
                           const double *val, int P, int R_max,
                           int32_t *hy_cnt, int32_t *hy_idx, double *hy_val,
                           uint8_t *route, int32_t *bk_rows, int32_t *bk_count)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int m = 0; m < M; ++m) {
        int nnz = 0, over = 0;
        for (int t = 0; t < NT; ++t) {
            const int c = cnt[(size_t)m * NT + t];
            nnz += c;
            if (c > C)
                over = 1;
        }
        hy_cnt[m] = nnz;
        route[m] = (uint8_t)(over || nnz > P);
        for (int s = 0; s < P; ++s) {
            hy_idx[(size_t)m * P + s] = -1;
            hy_val[(size_t)m * P + s] = 0.0;
        }
        if (route[m])
            continue;
        int n = 0;
        for (int t = 0; t < NT; ++t) {
            const size_t tile = (size_t)m * NT + t;
            for (int s = 0; s < cnt[tile]; ++s) {
                hy_idx[(size_t)m * P + n] = idx[tile * C + s];
                hy_val[(size_t)m * P + n] = val[tile * C + s];
                ++n;
            }
        }
    }
    int r = 0;
    for (int m = 0; m < M; ++m) {
        if (route[m]) {
            if (r < R_max)
                bk_rows[r] = m;
            ++r;
        }
    }
    *bk_count = r;
}

/* Up projection of the training forward in hybrid form: the dense-to-hybrid
 * product of section 3-7 (dense x times dense W_u, evaluated only where the
 * stored gate is non-zero), multiplied elementwise by the gate (section 1-1,
 * h = h_u h_g).  Sparse rows: for each stored entry s (column j, gate g),
 * hy_u = x_m . W_u[:, j] and hy_h = hy_u g.  The first nbk backup rows
 * (m = bk_rows[r]) are recomputed densely from x (section 3-6: heavy rows are
 * kept whole, not clipped): bk_g[r][j] = ReLU(x_m . W_g[:, j]),
 * bk_u[r][j] = x_m . W_u[:, j], bk_h = bk_u bk_g, for every j. */
void tw_oracle_hybrid_up(const double *x, const double *wg_t, const double *wu_t,
                         int M, int K, int N, int P,
                         const int32_t *hy_cnt, const int32_t *hy_idx, const double *hy_g,
                         const uint8_t *route, const int32_t *bk_rows, int nbk,
                         double *hy_u, double *hy_h, double *bk_g, double *bk_u, double *bk_h)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        if (route[m])
            continue;
        const double *xm = x + (size_t)m * K;
        for (int s = 0; s < hy_cnt[m]; ++s) {
            const size_t e = (size_t)m * P + s;
            const double u = dot(xm, wu_t + (size_t)hy_idx[e] * K, K);
            hy_u[e] = u;
            hy_h[e] = u * hy_g[e];
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nbk; ++r) {
        const double *xm = x + (size_t)bk_rows[r] * K;
        for (int j = 0; j < N; ++j) {
            const size_t e = (size_t)r * N + j;
            const double g = relu(dot(xm, wg_t + (size_t)j * K, K));
            const double u = dot(xm, wu_t + (size_t)j * K, K);
            bk_g[e] = g;
            bk_u[e] = u;
            bk_h[e] = u * g;
        }
    }
}

/* Down projection of the training forward: the hybrid-to-dense product of
 * section 3-7, y = h W_d with h in hybrid form.  A sparse row sums its
 * stored entries, y_m = sum over s of hy_h[s] W_d[hy_idx[s], :] (s
 * ascending); backup row r sums its dense row, y_m = sum over j ascending of
 * bk_h[r][j] W_d[j, :], for m = bk_rows[r], r < nbk.  Rows routed to the
 * backup but past nbk are not written. */
void tw_oracle_hybrid_down(const double *wd, int M, int K, int N, int P,
                           const int32_t *hy_cnt, const int32_t *hy_idx, const double *hy_h,
                           const uint8_t *route, const int32_t *bk_rows, int nbk,
                           const double *bk_h, double *y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        if (route[m])
            continue;
        double *ym = y + (size_t)m * K;
        for (int k = 0; k < K; ++k)
            ym[k] = 0.0;
        for (int s = 0; s < hy_cnt[m]; ++s) {
            const size_t e = (size_t)m * P + s;
            const double *wdj = wd + (size_t)hy_idx[e] * K;
            for (int k = 0; k < K; ++k)
                ym[k] += hy_h[e] * wdj[k];
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nbk; ++r) {
        double *ym = y + (size_t)bk_rows[r] * K;
        for (int k = 0; k < K; ++k)
            ym[k] = 0.0;
        for (int j = 0; j < N; ++j) {
            const double *wdj = wd + (size_t)j * K;
            for (int k = 0; k < K; ++k)
                ym[k] += bk_h[(size_t)r * N + j] * wdj[k];
        }
    }
}

/* Backward of the block over hybrid storage, section 3-7 (the gradients are
 * formed from the stored sparse activations without rebuilding the dense
 * hidden state), with the activation L1 penalty of section 3-2 injected into
 * the gate gradient.
 *
 * Given dy = dLoss/dy [M][K] and the forward's stored g (= h_g), u (= h_u)
 * and h = g u, by the chain rule through section 1-1's equation:
 *   dh[m][j]  = dy_m . W_d[j, :]                       (dense-to-hybrid)
 *   du[m][j]  = dh g                                    (gradient of h_u)
 *   dz[m][j]  = dh u + l1   where g > 0, else 0         (through the ReLU;
 *               l1 is the L1 penalty's gradient on a positive activation)
 *   dx_m      = sum_j du W_u[:, j]^T + dz W_g[:, j]^T   (hybrid-to-dense)
 *   dW_d[j]   = sum_m h[m][j] dy_m
 *   dW_u[:,j] = sum_m du[m][j] x_m,  dW_g[:,j] = sum_m dz[m][j] x_m
 * (the weight gradients read the stored activations column by column: the
 * hybrid transpose).  The transposed weight layouts hold dwu_t[j] = dW_u[:,j]
 * and dwg_t[j] = dW_g[:,j].  Sparse rows visit their stored entries in slot
 * order; the first nbk backup rows visit every column j in ascending order
 * (their dense g, u, h); other backup rows have no stored activation and
 * contribute nothing (dx rows left unwritten).  Weight-gradient sums run
 * over rows in ascending order. */
void tw_oracle_hybrid_bwd(const double *x, const double *wg_t, const double *wu_t,
                          const double *wd, const double *dy, int M, int K, int N, int P,
                          double l1, const int32_t *hy_cnt, const int32_t *hy_idx,
                          const double *hy_g, const double *hy_u, const double *hy_h,
                          const uint8_t *route, const int32_t *bk_rows, int nbk,
                          const double *bk_g, const double *bk_u, const double *bk_h,
                          double *hy_du, double *hy_dz, double *bk_du, double *bk_dz,
                          double *dx, double *dwg_t, double *dwu_t, double *dwd)
{
    /* gradients of the stored activations */
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        if (route[m])
            continue;
        const double *dym = dy + (size_t)m * K;
        for (int s = 0; s < hy_cnt[m]; ++s) {
            const size_t e = (size_t)m * P + s;
            const double dh = dot(dym, wd + (size_t)hy_idx[e] * K, K);
            hy_du[e] = dh * hy_g[e];
            hy_dz[e] = dh * hy_u[e] + l1;
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nbk; ++r) {
        const double *dym = dy + (size_t)bk_rows[r] * K;
        for (int j = 0; j < N; ++j) {
            const size_t e = (size_t)r * N + j;
            const double dh = dot(dym, wd + (size_t)j * K, K);
            bk_du[e] = dh * bk_g[e];
            bk_dz[e] = bk_g[e] > 0.0 ? dh * bk_u[e] + l1 : 0.0;
        }
    }
    /* input gradient */
#pragma omp parallel for schedule(dynamic, 1)
    for (int m = 0; m < M; ++m) {
        if (route[m])
            continue;
        double *dxm = dx + (size_t)m * K;
        for (int k = 0; k < K; ++k)
            dxm[k] = 0.0;
        for (int s = 0; s < hy_cnt[m]; ++s) {
            const size_t e = (size_t)m * P + s;
            const double *wu = wu_t + (size_t)hy_idx[e] * K;
            const double *wg = wg_t + (size_t)hy_idx[e] * K;
            for (int k = 0; k < K; ++k)
                dxm[k] += hy_du[e] * wu[k] + hy_dz[e] * wg[k];
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < nbk; ++r) {
        double *dxm = dx + (size_t)bk_rows[r] * K;
        for (int k = 0; k < K; ++k)
            dxm[k] = 0.0;
        for (int j = 0; j < N; ++j) {
            const size_t e = (size_t)r * N + j;
            const double *wu = wu_t + (size_t)j * K;
            const double *wg = wg_t + (size_t)j * K;
            for (int k = 0; k < K; ++k)
                dxm[k] += bk_du[e] * wu[k] + bk_dz[e] * wg[k];
        }
    }
    /* weight gradients: each thread owns a range of hidden columns and walks
     * every row in ascending order */
#pragma omp parallel
    {
#ifdef _OPENMP
        const int nt = omp_get_num_threads(), t = omp_get_thread_num();
#else
        const int nt = 1, t = 0;
#endif
        const int j0 = (int)((long long)N * t / nt), j1 = (int)((long long)N * (t + 1) / nt);
        for (size_t q = (size_t)j0 * K; q < (size_t)j1 * K; ++q) {
            dwd[q] = 0.0;
            dwu_t[q] = 0.0;
            dwg_t[q] = 0.0;
        }
        int r = 0;  /* next backup slot, in ascending row order */
        for (int m = 0; m < M; ++m) {
            const double *xm = x + (size_t)m * K;
            const double *dym = dy + (size_t)m * K;
            if (!route[m]) {
                for (int s = 0; s < hy_cnt[m]; ++s) {
                    const size_t e = (size_t)m * P + s;
                    const int j = hy_idx[e];
                    if (j < j0 || j >= j1)
                        continue;
                    for (int k = 0; k < K; ++k) {
                        dwd[(size_t)j * K + k] += hy_h[e] * dym[k];
                        dwu_t[(size_t)j * K + k] += hy_du[e] * xm[k];
                        dwg_t[(size_t)j * K + k] += hy_dz[e] * xm[k];
                    }
                }
            } else if (r < nbk && bk_rows[r] == m) {
                for (int j = j0; j < j1; ++j) {
                    const size_t e = (size_t)r * N + j;
                    for (int k = 0; k < K; ++k) {
                        dwd[(size_t)j * K + k] += bk_h[e] * dym[k];
                        dwu_t[(size_t)j * K + k] += bk_du[e] * xm[k];
                        dwg_t[(size_t)j * K + k] += bk_dz[e] * xm[k];
                    }
                }
                ++r;
            }
        }
    }
}
