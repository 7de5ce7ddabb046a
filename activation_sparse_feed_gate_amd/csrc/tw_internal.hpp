// tw_internal.hpp -- launchers of the gfx950 kernels behind the C ABI.
// Every launcher only enqueues work on `s` and returns the launch status; the
// C ABI layer validates all arguments before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tw {

// Gate GEMM macro tile: 256 token rows x 256 hidden columns.
constexpr int kGateBM = 256;
constexpr int kGateBN = 256;

inline int gate_col_blocks(int N) { return (N + kGateBN - 1) / kGateBN; }
inline int row_words(int M) { return (M + 31) / 32; }

// Whether a batch of M rows takes the small-batch gate kernel (64-row tiles
// of one TwELL tile each): while the 256 x 256 macro tiles would number
// fewer than 64 (measured crossover).  Its row-overflow bits come in N / T
// column blocks instead of N / 256.
inline bool gate_small(int M, int N) {
    return (long long)((M + kGateBM - 1) / kGateBM) * gate_col_blocks(N) < 64;
}
// Column blocks of the row-overflow bits launch_gate_twell writes.
int gate_flag_blocks(int M, int N, int T);

// Workspace of the small-batch gate's split reduction (fp32 partial gates;
// 0 when the batch does not take it).
size_t gate_part_bytes(int M, int K, int N);

hipError_t launch_gate_twell(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N,
                             int T, int C, float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                             uint32_t *oflag, float *z_debug, float *part, hipStream_t s);

// The dense gate z = x W_g as fp32 [M][N] (the gate kernel without its
// packing epilogue).
hipError_t launch_gate_dense(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N,
                             float *z, hipStream_t s);

// TwELL packing and row-overflow bits of a dense gate [M][N], in the same
// layouts the fused gate kernel writes (the compaction follows).
hipError_t launch_pack_dense(const float *z, int M, int N, int T, int C, float *tw_val,
                             int32_t *tw_idx, int32_t *tw_cnt, uint32_t *oflag, hipStream_t s);

hipError_t launch_ovf_compact(const uint32_t *oflag, int NB, int MW, int R_max,
                              int32_t *ovf_rows, int32_t *ovf_count, hipStream_t s);

// Workgroups per row of the sparse kernel: batches of 32 to 128 rows are
// spread over G = 256 / M per row, which write partial rows
// (sparse_rowpart_bytes of them) that a second kernel sums; else 1.
// Measured: below 32 rows the second kernel costs more than the split
// gains, and 512 / M parts were slower at the 0.5B block shape.
inline int sparse_row_parts(int M) {
    if (M < 32 || M > 128) return 1;
    return 256 / M;
}
inline size_t sparse_rowpart_bytes(int M, int K) {
    const int g = sparse_row_parts(M);
    return g > 1 ? (size_t)g * M * K * 4 : 0;
}

// Heaviest-first dispatch of the sparse kernel.  A row's gathers form a
// serial chain per wave, so a heavy row that starts late sets the kernel's
// end.  The rows are cut into segments of kOrderSeg; for each segment one
// extra workgroup of the overflow rows' gate+up launch (running beside the
// GEMM) lists its rows with no tile over capacity and more than H entries,
// then its other rows, each ascending, and counts both.  Workgroup b of the
// sparse kernel takes the b-th row of the order "every segment's heavy
// rows, then every segment's other rows", located by a scan of the counts.
// perm layout: int32 heavy counts [64], other counts [64], then M row slots
// (segment s at s * kOrderSeg).
struct RowOrder {
    const int32_t *tw_cnt = nullptr;  // [M][NT]
    int M = 0, NT = 0, C = 0, H = 0;
    int32_t *perm = nullptr;          // null: no ordering
};
constexpr int kOrderSeg = 256;
__host__ __device__ inline int row_order_segs(int M) { return (M + kOrderSeg - 1) / kOrderSeg; }
inline size_t row_order_bytes(int M) { return 512 + (size_t)M * 4; }
// Batches that take it: more than 256 rows (one workgroup per row) and at
// most kHeavyFirstRows.  Measured (sparse kernel, unordered against
// ordered): 38.4 against 32.8 us at the 0.5B block, 63.5 against 53.9 at
// the paper shape, 87.9 against 79.9 at the 1B block; at 16384 rows, where
// the kernel streams near the HBM rate, 236.9 against 242.2 (2B block) and
// 77.3 against 86.9 (overflow-stress block).
constexpr int kHeavyFirstRows = 8192;
static_assert(kHeavyFirstRows <= 64 * kOrderSeg, "the counts of 64 segments");
inline bool sparse_heavy_first(int M) { return M > 256 && M <= kHeavyFirstRows; }
// A row is heavy with more than this many entries (measured 32.8 us at the
// 0.5B block against 33.4 with 32 and 34.4 with 16).
constexpr int kHeavyEntries = 64;

// Sparse up + down of every non-overflow row into y.  With `partial` (the
// split partial tiles launch_down left for the overflow list ovf_rows,
// ovf_count, R_max), it also sums those into the listed rows of y, in place
// of launch_split_reduce; partial null: overflow rows are left alone.
// rowpart: sparse_rowpart_bytes(M, K) bytes (unused when that is 0).
// perm: the heaviest-first row order (RowOrder), or null for row order.
hipError_t launch_sparse_updown(const uint16_t *x, const uint16_t *wu_t, const uint16_t *wd,
                                int M, int K, int N, int T, int C, const float *tw_val,
                                const int32_t *tw_idx, const int32_t *tw_cnt, float *y,
                                const float *partial, const int32_t *ovf_rows,
                                const int32_t *ovf_count, int R_max, float *rowpart,
                                const int32_t *perm, hipStream_t s);

// Row-list gate+up GEMMs with a capacity of at most this many rows take
// 128-row x 64-column tiles (256 of them at this capacity; 64 x 64 tiles up
// to 64 rows of capacity), larger row lists 128 x 128 tiles.  The row count itself is known only on the device; with
// the usual capacity of an eighth of the batch the small tiles measured
// faster below about 400 listed rows and 128 x 128 tiles above (at 360-1000
// rows the larger tiles took 25-40% less time than 64 x 64 ones).
constexpr int kSmallRows = 512;
// Whether the all-rows down GEMM of M rows splits its reduction (too few
// output tiles to fill the chip); it then needs split_partial_bytes().
bool dense_down_split(int M, int K);

// h[r][n] = bf16(ReLU(x_r . wg_t[n]) * (x_r . wu_t[n])) for r < rows, where
// x_r is x[rowlist[r]] (rowlist != nullptr, rows = min(*count, R_cap)) or
// x[r] (rowlist == nullptr, rows = R_cap).  x has M rows; with a row list
// M * K * 2 must stay below 4 GiB (32-bit buffer offsets).
// With ord.perm (row lists only) one more workgroup writes the sparse
// kernel's heaviest-first row order.
hipError_t launch_gateup(const uint16_t *x, int M, const uint16_t *wg_t, const uint16_t *wu_t,
                         int K, int N, const int32_t *rowlist, const int32_t *count,
                         int R_cap, uint16_t *h, hipStream_t s, const RowOrder &ord = RowOrder());

// launch_gateup over a row list that also stores g_out[r][n] =
// bf16(ReLU(x_r . wg_t[n])) and u_out[r][n] = bf16(x_r . wu_t[n]) where
// those are non-null.
hipError_t launch_gateup_keep(const uint16_t *x, int M, const uint16_t *wg_t,
                              const uint16_t *wu_t, int K, int N, const int32_t *rowlist,
                              const int32_t *count, int R_cap, uint16_t *h, uint16_t *g_out,
                              uint16_t *u_out, hipStream_t s);

// Backward of the backup rows' activations: dh = dy_r . wd[n] on the matrix
// cores (one weight operand), then du[r][n] = bf16(dh g) and dz[r][n] =
// bf16(g > 0 ? dh u + l1 : 0) with the row's stored bf16 g_in, u_in.
hipError_t launch_backup_dh(const uint16_t *dy, int M, const uint16_t *wd, int K, int N,
                            const int32_t *rowlist, const int32_t *count, int R_cap,
                            const uint16_t *g_in, const uint16_t *u_in, float l1,
                            uint16_t *du, uint16_t *dz, hipStream_t s);

// y[row_r][k] = sum_n h[r][n] * wd[n][k] (fp32) for r < rows, with row_r =
// rowlist[r] or r as above.  With a `partial` buffer (split_partial_bytes())
// the reduction is split when there are few rows, and launch_split_reduce
// must follow on the stream to sum the partial tiles into y.
hipError_t launch_down(const uint16_t *h, const uint16_t *wd, int K, int N,
                       const int32_t *rowlist, const int32_t *count, int R_cap, float *y,
                       float *partial, hipStream_t s);
hipError_t launch_split_reduce(const float *partial, const int32_t *rowlist,
                               const int32_t *count, int R_cap, int K, int N, float *y,
                               hipStream_t s);
size_t split_partial_bytes();
// y[row_r] = h[r] W_d + h2[r] W_d2 for r < rows (row list as above): one
// GEMM whose reduction runs over both products (2 N deep), split as
// launch_down splits; launch_split_reduce with 2 N, or launch_hybrid_dx,
// sums the partial tiles.
hipError_t launch_down_pair(const uint16_t *h, const uint16_t *wd, const uint16_t *h2,
                            const uint16_t *wd2, int K, int N, const int32_t *rowlist,
                            const int32_t *count, int R_cap, float *y, float *partial,
                            hipStream_t s);

// Hybrid storage of the training forward (hybrid.hip).
hipError_t launch_hybrid_pack(const float *tw_val, const int32_t *tw_idx, const int32_t *tw_cnt,
                              int M, int N, int T, int C, int P, float *hy_val, int32_t *hy_idx,
                              int32_t *hy_cnt, uint8_t *route, hipStream_t s);
hipError_t launch_route_compact(const uint8_t *route, int M, int R_max, int32_t *bk_rows,
                                int32_t *bk_count, hipStream_t s);
hipError_t launch_hybrid_up(const uint16_t *x, const uint16_t *wu_t, int M, int K, int N, int P,
                            const float *hy_g, const int32_t *hy_idx, const int32_t *hy_cnt,
                            const uint8_t *route, float *hy_u, float *hy_h, hipStream_t s);
// With `partial` (the split partial tiles launch_down or launch_down_pair
// left for the backup list bk_rows, bk_count, R_max), the kernel also sums
// those into the listed rows, in place of launch_split_reduce.
hipError_t launch_hybrid_down(const uint16_t *wd, int M, int K, int N, int P, const float *hy_h,
                              const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                              float *y, const float *partial, const int32_t *bk_rows,
                              const int32_t *bk_count, int R_max, hipStream_t s);
// Backward over hybrid storage: du, dz at the stored entries of sparse rows;
// dx of sparse rows; the transpose and weight gradients (all rows).
hipError_t launch_hybrid_dh(const uint16_t *dy, const uint16_t *wd, int M, int K, int N, int P,
                            const float *hy_g, const float *hy_u, float l1, const int32_t *hy_idx,
                            const int32_t *hy_cnt, const uint8_t *route, float *hy_du,
                            float *hy_dz, hipStream_t s);
hipError_t launch_hybrid_dx(const uint16_t *wu_t, const uint16_t *wg_t, int M, int K, int N,
                            int P, const float *hy_du, const float *hy_dz,
                            const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                            float *dx, const float *partial, const int32_t *bk_rows,
                            const int32_t *bk_count, int R_max, hipStream_t s);
size_t hybrid_dw_bytes(int M, int K, int N, int P, int R_max);
hipError_t launch_hybrid_dw(const uint16_t *x, const uint16_t *dy, int M, int K, int N, int P,
                            const float *hy_h, const float *hy_du, const float *hy_dz,
                            const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                            const int32_t *bk_rows, const int32_t *bk_count, int R_max,
                            const uint16_t *bk_h, const uint16_t *bk_du, const uint16_t *bk_dz,
                            float *dwg_t, float *dwu_t, float *dwd, void *ws, hipStream_t s,
                            hipEvent_t ev_transposed, hipEvent_t ev_sparse);
// Weight gradients of the backup rows, added into dwd / dwu_t / dwg_t:
// dwd += bk_h^T dy_bk, dwu_t += bk_du^T x_bk, dwg_t += bk_dz^T x_bk, with the
// rows' dy and x first gathered into dy_bk / x_bk (backup_gather_bytes each).
size_t backup_gather_bytes(int R_max, int K);
hipError_t launch_backup_wgrad(const uint16_t *dy, const uint16_t *x, int K, int N,
                               const int32_t *rowlist, const int32_t *count, int R_cap,
                               const uint16_t *bk_h, const uint16_t *bk_du,
                               const uint16_t *bk_dz, uint16_t *dy_bk, uint16_t *x_bk,
                               float *dwd, float *dwu_t, float *dwg_t, hipStream_t s);

}  // namespace tw
