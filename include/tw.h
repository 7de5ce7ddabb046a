/*
 * tw.h -- C ABI of the TwELL sparse gated-FFN forward for AMD MI355X (gfx950).
 *
 * The block computed is the ReLU-gated feed-forward layer of "Sparser,
 * Faster, Lighter Transformer Language Models Review", section 1-1:
 *
 *     h_u = x W_u,   h_g = ReLU(x W_g),   h = h_u (elementwise) h_g,   y = h W_d
 *
 * with x [M, K] (M tokens, model dimension K) and an expanded hidden
 * dimension N.  Its two-stage inference path (section 2-2: a gate projection
 * whose epilogue builds the packed form, then the up and down projections
 * fused over the active neurons) is split over two calls:
 *
 *   tw_pack_gate       gate GEMM whose epilogue applies the ReLU and packs the
 *                      active entries of every (token row, column tile) in the
 *                      tile-wise ELLPACK layout of section 3-4, and builds the
 *                      list of rows that overflow a tile's capacity
 *                      (the dense-backup routing of sections 3-6 and 4-3);
 *   tw_sparse_ffn_fwd  per-token sparse up+down (section 3-5 equation) for the
 *                      rows that fit, and the dense path for the listed rows.
 *
 * tw_ffn_fwd is the dense gated FFN over all rows, the comparator the sparse
 * path is measured against.  tw_gate_dense + tw_pack_dense are the unfused
 * equivalent of tw_pack_gate (dense gate written to memory, then packed).
 * tw_hybrid_pack, tw_hybrid_up and tw_hybrid_down are the training forward
 * over the hybrid storage of sections 3-6 and 3-7, and tw_hybrid_bwd_dh,
 * tw_hybrid_bwd_dx and tw_hybrid_bwd_dw its backward (declared at the end).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - bf16 values travel as raw uint16_t bit patterns.
 * - Every pointer argument except `stream` is a device pointer to memory the
 *   caller owns.  The library allocates no device memory and keeps no
 *   state between calls, so calls on different streams may run
 *   concurrently as long as their output and workspace buffers are
 *   distinct.  The one exception is tw_pack_gate_noalloc, whose workspace
 *   is a static device array inside the library, shared by every call on
 *   one GPU (see its declaration).
 * - All work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *   void*; NULL is the default stream).  Nothing synchronises the host.
 * - Argument and shape errors are detected on the host before any work is
 *   enqueued and return TW_EINVAL or TW_EUNSUPPORTED; no output is touched
 *   then.  A failed kernel launch returns TW_EHIP.  tw_last_error() gives a
 *   message for the last failure of the calling thread.
 * - Device buffers must be 16-byte aligned.  When M == 0 the buffers whose
 *   size is a multiple of M may be NULL.
 * - Optional `events`: NULL, or an array of hipEvent_t (passed as void*)
 *   with one more entry than the call launches kernels, for per-kernel
 *   durations with hipEventElapsedTime.  tw_pack_gate records events[0]
 *   on `stream` before the gate, events[1] after it (one kernel; for a few
 *   token rows two: the K-sliced partial gates, then their sum and the
 *   packing) and events[2] after the overflow-list compaction.  tw_ffn_fwd
 *   (2 kernels) records events[0] before the first kernel and events[i+1]
 *   after kernel i.  tw_sparse_ffn_fwd takes 5
 *   events for 3 kernels: events[0] before any of them, events[1] and [2]
 *   after the overflow rows' gate+up and down GEMMs, events[3] after the
 *   sparse up+down kernel (which also finishes the overflow rows' split
 *   sums; for batches of 32 to 128 rows it is followed by the sum of its
 *   partial rows), events[4] together with events[3] (with R_max == 0 only
 *   the sparse kernel runs and events[0..2] are recorded together).
 *
 * Weight layout (one layout serves every path): wg_t, wu_t and wd are all
 * [N][K] row-major bf16.  wg_t and wu_t hold W_g and W_u transposed, so the
 * weights of hidden neuron j (column j of W_g / W_u) are row j, contiguous;
 * wd is W_d itself, whose row j is what neuron j adds to the output.
 *
 * Supported shapes: M >= 0, K a positive multiple of 128 and at most 4096,
 * N a positive multiple of T, T in {128, 256}, N / T <= 256, 1 <= C <= T,
 * 0 <= R_max <= M, and M * K < 2^31 (x under 4 GiB: the dense backup
 * gathers its rows with 32-bit buffer offsets).  tw_ffn_fwd has its own
 * limits, stated at its declaration.
 */
#ifndef TW_H
#define TW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tw_status {
    TW_OK = 0,
    TW_EINVAL = 1,        /* null pointer, bad size, misaligned buffer     */
    TW_EUNSUPPORTED = 2,  /* valid but outside the supported shapes above  */
    TW_EHIP = 3           /* a HIP runtime call or kernel launch failed    */
} tw_status;

/* Static name of a status code. */
const char *tw_status_str(int status);

/* Message describing the last non-OK status returned on the calling thread
 * (empty string if none). */
const char *tw_last_error(void);

/* Bytes of device workspace tw_pack_gate and tw_sparse_ffn_fwd need for
 * this shape (one buffer of this size serves both); 0 for arguments that
 * the entry points would reject. */
size_t tw_workspace_bytes(int M, int K, int N, int T, int C, int R_max);

/*
 * Gate GEMM + ReLU + TwELL packing + overflow routing.
 *
 * Computes z = x W_g in fp32 (bf16 products, fp32 accumulation) and, for
 * every token row m and column tile t (columns [t*T, (t+1)*T)):
 *   tw_cnt[m][t]          number of columns j in the tile with z[m][j] > 0
 *                         (strictly positive; the true count, even above C)
 *   tw_idx[m][t][s]       the s-th such j, ascending, as a global column
 *   tw_val[m][t][s]       z[m][j] (fp32) for that j
 * for s < min(tw_cnt[m][t], C); slots from min(cnt, C) to C-1 are left
 * untouched.  These are the packed values, original hidden indices and
 * per-(row, tile) counts of section 3-4 (h_v, h_I, h_nz).
 *
 * A row with any tile holding more than C active columns overflows and is
 * routed whole to the dense path (sections 3-6 and 4-3): ovf_rows receives
 * the overflowing rows in ascending order, at most R_max of them, and
 * *ovf_count their true number.  *ovf_count > R_max means that the rows past
 * the first R_max will not be recomputed: read ovf_count after the stream
 * has run and retry with a larger R_max (or C) -- the retry of section 4-3.
 *
 *   x        [M][K]          bf16, token rows
 *   wg_t     [N][K]          bf16, W_g transposed
 *   tw_val   [M][N/T][C]     fp32 out
 *   tw_idx   [M][N/T][C]     int32 out
 *   tw_cnt   [M][N/T]        int32 out
 *   ovf_rows [max(R_max,1)]  int32 out
 *   ovf_count[1]             int32 out
 *   z_debug  [M][N]          fp32 out, or NULL; receives z itself (the same
 *                            values the packing used) -- for tests
 *   ws       workspace of ws_bytes >= tw_workspace_bytes(M, K, N, T, C, R_max)
 *
 * ovf_rows and ovf_count may both be NULL (one alone is TW_EINVAL): then no
 * overflow list is built and the compaction kernel does not run (events[2]
 * is recorded right after events[1]).  tw_sparse_ffn_fwd needs the list;
 * the training path does not (tw_hybrid_pack routes rows from tw_cnt).
 */
tw_status tw_pack_gate(const uint16_t *x, const uint16_t *wg_t,
                       int M, int K, int N, int T, int C,
                       float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                       int32_t *ovf_rows, int32_t *ovf_count, int R_max,
                       float *z_debug, void *ws, size_t ws_bytes,
                       void *stream, void *const *events);

/*
 * tw_pack_gate without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same kernels, arguments, outputs and
 * error behaviour as tw_pack_gate; the workspace is instead a static device
 * array inside the library of 16 MiB per GPU (held by every GPU the library
 * runs on until the process ends; its address is looked up once per device,
 * on the first call there).  Shapes whose tw_pack_gate workspace would
 * exceed it (row-overflow bits of (N/128) * ceil(M/32) words, plus for a few
 * token rows the small-batch gate's partial gates) return TW_EUNSUPPORTED
 * with a message giving the bytes needed.  The call allocates nothing.  All
 * calls on one GPU share that GPU's array, so calls that overlap on one GPU
 * (on two streams, or from two host threads) race; calls in stream order do
 * not.  Nothing in the array needs to start at zero.
 */
tw_status tw_pack_gate_noalloc(const uint16_t *x, const uint16_t *wg_t,
                               int M, int K, int N, int T, int C,
                               float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                               int32_t *ovf_rows, int32_t *ovf_count, int R_max,
                               float *z_debug, void *stream, void *const *events);

/*
 * The unfused alternative to tw_pack_gate, in two calls: section 3-4
 * contrasts packing in the gate's epilogue with computing the dense gate,
 * writing it to memory and packing it in a separate pass (an extra write,
 * read and write of the whole gate).  These calls are that separate path,
 * kept for measuring what the fusion saves and for packing gates computed
 * elsewhere; their outputs are identical to tw_pack_gate's.
 *
 * tw_gate_dense: z = x W_g as fp32 [M][N] (the same kernel and arithmetic
 * as tw_pack_gate, so z is bitwise tw_pack_gate's z_debug).  K and N
 * multiples of 128, K <= 4096, M * K < 2^31 (tw_pack_gate's limits; other
 * shapes return TW_EUNSUPPORTED).  events: [0] before, [1] after the kernel.
 *
 * tw_pack_dense: TwELL packing and overflow routing of any fp32 gate z
 * [M][N] (active means z > 0), with exactly the outputs and conventions of
 * tw_pack_gate above (same shape limits on N, T, C, R_max).  The workspace
 * holds the row-overflow bits: ws_bytes >= tw_pack_dense_workspace_bytes
 * (tw_workspace_bytes of the same shape is always enough).  events: [0]
 * before, [1] after the packing kernel, [2] after the compaction.
 */
tw_status tw_gate_dense(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N, float *z,
                        void *stream, void *const *events);
size_t tw_pack_dense_workspace_bytes(int M, int N);
tw_status tw_pack_dense(const float *z, int M, int N, int T, int C,
                        float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                        int32_t *ovf_rows, int32_t *ovf_count, int R_max,
                        void *ws, size_t ws_bytes, void *stream, void *const *events);

/*
 * Sparse up+down for the rows that fit, dense path for the overflow list.
 *
 * For every row m with no tile over capacity (every tw_cnt[m][t] <= C), with
 * the packed (j, g) pairs of tw_pack_gate:
 *     y[m][:] = sum over packed (j, g) of (x[m] . Wu_t[j]) * g * Wd[j][:]
 * (section 3-5 equation; the up activation is a scalar per active neuron,
 * fp32 throughout).  A row with no active neuron gets y = 0.
 * For r < min(*ovf_count, R_max), the row m = ovf_rows[r] gets the dense
 * gated FFN of section 1-1 instead (h rounded to bf16 before W_d, fp32
 * accumulation).  Rows that overflow but lie past R_max are left untouched.
 *
 *   x, wg_t, wu_t, wd       as above ([M][K] and [N][K] bf16)
 *   tw_val, tw_idx, tw_cnt  the packing written by tw_pack_gate
 *   ovf_rows, ovf_count     the routing written by tw_pack_gate (device)
 *   y        [M][K]         fp32 out
 *
 * On `stream`, the overflow rows' dense path runs first: gate+up, then the
 * down GEMM, which for few rows splits its reduction over N into partial
 * tiles in the workspace.  The sparse kernel follows; it computes the rows
 * that fit and sums those partials (in split order, so the result does not
 * depend on timing) into the listed rows.  The two sets of rows are
 * disjoint.  Batches of 32 to 128 rows spread each row over several
 * workgroups, whose partial rows (in the workspace) a last small kernel
 * sums in a fixed order.  Batches of 257 to 8192 rows (with R_max > 0)
 * start their heaviest rows first, in an order that extra workgroups of the
 * gate+up launch write to the workspace from tw_cnt; each row is still
 * computed once by the same code, so y does not depend on the order.
 */
tw_status tw_sparse_ffn_fwd(const uint16_t *x, const uint16_t *wg_t,
                            const uint16_t *wu_t, const uint16_t *wd,
                            int M, int K, int N, int T, int C,
                            const float *tw_val, const int32_t *tw_idx,
                            const int32_t *tw_cnt, const int32_t *ovf_rows,
                            const int32_t *ovf_count, int R_max,
                            float *y, void *ws, size_t ws_bytes,
                            void *stream, void *const *events);

/*
 * Dense gated FFN over all M rows (section 1-1 equation): the gate and up
 * projections in one MFMA GEMM whose epilogue forms h = ReLU(g) * u rounded
 * to bf16, then the down projection into fp32 y [M][K] (when M is too small
 * for its output tiles to fill the chip, split over N and summed by a
 * second kernel; events[2] follows both).  The workspace holds h [M][N]
 * bf16 and, when the down projection splits, the partial sums:
 * ws_bytes >= tw_ffn_workspace_bytes.
 * Shapes: M >= 0, K and N positive multiples of 128, N * K < 2^31 (each
 * weight matrix under 4 GiB: 32-bit buffer offsets).  The workspace query
 * returns 0 for any other shape.
 */
size_t tw_ffn_workspace_bytes(int M, int K, int N);
tw_status tw_ffn_fwd(const uint16_t *x, const uint16_t *wg_t,
                     const uint16_t *wu_t, const uint16_t *wd,
                     int M, int K, int N, float *y, void *ws, size_t ws_bytes,
                     void *stream, void *const *events);

/*
 * Hybrid storage for the training forward (sections 3-6, 3-7 and 4-3).
 *
 * Training keeps the gate activation in a hybrid form built from the TwELL
 * gate (section 2-2: TwELL gate, then hybrid storage): most token rows as a
 * row-wide ELL of at most P entries (the values and original hidden indices
 * of section 3-3's ELL, in ascending column order), the few heavy rows whole
 * in a dense backup, and a binary routing vector saying which holds each
 * row.  The up and down projections then run as two separate products that
 * keep that form (section 3-7: in training they are not fused): the
 * dense-to-hybrid product (x W_u evaluated only at the stored entries, times
 * the gate) and the hybrid-to-dense product (h W_d).  The section 4-3
 * capacities are P = 128 stored entries per row and a backup of at most
 * M / 8 rows; an overflow of the backup is reported for a retry.
 *
 * Common arrays (device, caller-owned, P the sparse row capacity):
 *   hy_cnt  [M]        int32  the row's number of active neurons (the true
 *                             count, also for backup rows)
 *   hy_idx  [M][P]     int32  stored hidden index j of entry s < hy_cnt[m]
 *   hy_val / hy_u / hy_h [M][P]  fp32  gate value, up value, product of entry s
 *   route   [M]        uint8  1 if row m lives in the dense backup, else 0
 *   bk_rows [max(R_max,1)] int32  backup rows, ascending; slot r holds row bk_rows[r]
 *   bk_count[1]        int32  the true number of backup rows (may exceed R_max)
 *   bk_g / bk_u / bk_h [R_max][N] bf16  dense gate, up, product of backup slot r
 * Slots s >= hy_cnt[m] of a sparse row, and every slot of a backup row, are
 * left untouched.  A backup row past R_max (bk_count > R_max) is in neither
 * store: read bk_count after the stream has run and retry with a larger
 * R_max (or P) -- the retry of section 4-3.  Such rows get no output from
 * tw_hybrid_up or tw_hybrid_down.
 *
 * Shapes: as for tw_pack_gate (T in {128, 256}, N a multiple of T, N/T <=
 * 256, 1 <= C <= T, K a multiple of 128 and at most 4096, M*K < 2^31), and
 * N a multiple of 128, 1 <= P <= N, 0 <= R_max <= M, N*K < 2^31,
 * R_max*N < 2^31, and M*P < 2^31 (the kernels name a stored slot by the
 * 32-bit id m*P + s); other shapes return TW_EUNSUPPORTED.
 */

/*
 * TwELL -> hybrid.  Reads a TwELL packing of capacity C (tw_pack_gate's or
 * tw_pack_dense's outputs).  Row m goes to the dense backup when its total
 * count exceeds P or when one of its tiles held more than C entries (its
 * TwELL slots then lack entries); otherwise its TwELL entries are copied to
 * hy_idx / hy_val in ascending column order.  Writes hy_cnt, route and the
 * backup list.  The backup rows' dense values are produced by tw_hybrid_up.
 * events: [0] before, [1] after the packing kernel, [2] after the list.
 */
tw_status tw_hybrid_pack(int M, int N, int T, int C,
                         const float *tw_val, const int32_t *tw_idx, const int32_t *tw_cnt,
                         int P, float *hy_val, int32_t *hy_idx, int32_t *hy_cnt,
                         uint8_t *route, int32_t *bk_rows, int32_t *bk_count, int R_max,
                         void *stream, void *const *events);

/*
 * Dense-to-hybrid product of the up projection, times the gate.
 * Sparse rows: for each stored entry s (hidden index j, gate g = hy_g),
 *     hy_u[m][s] = x[m] . wu_t[j]   (fp32),   hy_h[m][s] = hy_u[m][s] * g.
 * Backup slots r < min(*bk_count, R_max), row m = bk_rows[r], all N columns
 * on the matrix cores (one GEMM over W_g and W_u, x read once):
 *     bk_g[r] = bf16(ReLU(x[m] W_g)),  bk_u[r] = bf16(x[m] W_u),
 *     bk_h[r] = bf16(ReLU(x[m] W_g) * (x[m] W_u))  (product before rounding).
 * hy_u, bk_g and bk_u may be NULL (not stored); hy_h and bk_h are required.
 * events: [0] before, [1] after the sparse-row kernel, [2] after the backup GEMM.
 */
tw_status tw_hybrid_up(const uint16_t *x, const uint16_t *wg_t, const uint16_t *wu_t,
                       int M, int K, int N, int P,
                       const float *hy_g, const int32_t *hy_idx, const int32_t *hy_cnt,
                       const uint8_t *route, const int32_t *bk_rows, const int32_t *bk_count,
                       int R_max, float *hy_u, float *hy_h,
                       uint16_t *bk_g, uint16_t *bk_u, uint16_t *bk_h,
                       void *stream, void *const *events);

/*
 * Hybrid-to-dense product of the down projection, y = h W_d (fp32 [M][K]).
 * Sparse rows: y[m] = sum over stored s of hy_h[m][s] * wd[hy_idx[m][s]]
 * (a row with no entry gets 0).  Backup slots r < min(*bk_count, R_max): the
 * row bk_rows[r] of y gets bk_h[r] W_d on the matrix cores.  The workspace
 * holds the backup GEMM's partial tiles: ws_bytes >=
 * tw_hybrid_down_workspace_bytes(R_max) (ws may be NULL when that is 0).
 * The backup GEMM runs first; the sparse-row kernel follows and also sums
 * the GEMM's partial tiles into the backup rows (in split order).
 * events: [0] before, [1] after the backup GEMM, [2] and [3] after the
 * sparse-row kernel.
 */
size_t tw_hybrid_down_workspace_bytes(int R_max);
tw_status tw_hybrid_down(const uint16_t *wd, int M, int K, int N, int P,
                         const float *hy_h, const int32_t *hy_idx, const int32_t *hy_cnt,
                         const uint8_t *route, const int32_t *bk_rows, const int32_t *bk_count,
                         int R_max, const uint16_t *bk_h, float *y,
                         void *ws, size_t ws_bytes, void *stream, void *const *events);

/*
 * Backward over the hybrid storage (section 3-7: the gradients are formed
 * from the stored sparse activations, without rebuilding a dense hidden
 * state; L1 gradient injection; the hybrid transpose for the weight
 * gradients), for the forward of tw_hybrid_pack / tw_hybrid_up /
 * tw_hybrid_down with g, u (hy_u, bk_g, bk_u) kept.  With dy = dLoss/dy
 * [M][K] (bf16) and the L1 penalty of section 3-2 on the gate activation,
 * whose gradient on a positive activation is the caller's `l1` (lambda
 * divided by the layer count and M N, in the pages' normalisation):
 *   dh = dy W_d^T,   du = dh g,   dz = (dh u + l1) where g > 0, else 0,
 *   dx = du W_u^T + dz W_g^T,
 *   dwd[j] = sum_m h[m][j] dy[m],  dwu_t[j] = sum_m du[m][j] x[m],
 *   dwg_t[j] = sum_m dz[m][j] x[m]
 * (dwu_t, dwg_t: gradients of W_u and W_g in their transposed [N][K] layout,
 * dwd of W_d [N][K]; all fp32).  Rows routed to the backup but past its room
 * (bk_count > R_max) stored nothing: they get no dx and add nothing to the
 * weight gradients.  Shapes as for the hybrid forward.
 *
 * tw_hybrid_bwd_dh (dense-to-hybrid): hy_du, hy_dz [M][P] fp32 at the stored
 * entries of sparse rows; bk_du, bk_dz [R_max][N] bf16 for backup slots (on
 * the matrix cores, from the row's stored bf16 bk_g, bk_u).  events: [0]
 * before, [1] after the sparse-row kernel, [2] after the backup GEMM.
 */
tw_status tw_hybrid_bwd_dh(const uint16_t *dy, const uint16_t *wd, int M, int K, int N, int P,
                           float l1, const float *hy_g, const float *hy_u, const int32_t *hy_idx,
                           const int32_t *hy_cnt, const uint8_t *route, const int32_t *bk_rows,
                           const int32_t *bk_count, int R_max, const uint16_t *bk_g,
                           const uint16_t *bk_u, float *hy_du, float *hy_dz, uint16_t *bk_du,
                           uint16_t *bk_dz, void *stream, void *const *events);

/*
 * tw_hybrid_bwd_dx (hybrid-to-dense): dx [M][K] fp32 for sparse rows and the
 * listed backup rows (the latter on the matrix cores: one GEMM whose
 * reduction runs over both products, du W_u^T then dz W_g^T, split into
 * partial tiles that the sparse-row kernel, which runs after it, sums in
 * split order).  ws_bytes >= tw_hybrid_bwd_dx_workspace_bytes(R_max) (ws
 * may be NULL when that is 0).  events: [0] before, [1] after the backup
 * GEMM, [2] after the sparse-row kernel.
 */
size_t tw_hybrid_bwd_dx_workspace_bytes(int R_max);
tw_status tw_hybrid_bwd_dx(const uint16_t *wg_t, const uint16_t *wu_t, int M, int K, int N, int P,
                           const float *hy_du, const float *hy_dz, const int32_t *hy_idx,
                           const int32_t *hy_cnt, const uint8_t *route, const int32_t *bk_rows,
                           const int32_t *bk_count, int R_max, const uint16_t *bk_du,
                           const uint16_t *bk_dz, float *dx, void *ws, size_t ws_bytes,
                           void *stream, void *const *events);

/*
 * tw_hybrid_bwd_dw: the three weight gradients, every row of dwg_t, dwu_t
 * and dwd written.  The sparse rows' part goes through the hybrid transpose
 * kept in the workspace: their stored entries grouped by hidden column in
 * ascending row order, so each column's gradient is a fixed-order sum; the
 * listed backup rows' part is three products on the matrix cores
 * (dwd += bk_h^T dy, dwu_t += bk_du^T x, dwg_t += bk_dz^T x over the backup
 * slots).  Results are bit-identical run to run.  ws_bytes >=
 * tw_hybrid_bwd_dw_workspace_bytes(M, K, N, P, R_max) (about 16 M P +
 * 4 R_max K bytes; 0 for a shape this call rejects).  events: [0] before,
 * [1] after the
 * transpose, [2] after the sparse rows' gradients, [3] after the backup
 * rows' products.
 */
size_t tw_hybrid_bwd_dw_workspace_bytes(int M, int K, int N, int P, int R_max);
tw_status tw_hybrid_bwd_dw(const uint16_t *x, const uint16_t *dy, int M, int K, int N, int P,
                           const float *hy_h, const float *hy_du, const float *hy_dz,
                           const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                           const int32_t *bk_rows, const int32_t *bk_count, int R_max,
                           const uint16_t *bk_h, const uint16_t *bk_du, const uint16_t *bk_dz,
                           float *dwg_t, float *dwu_t, float *dwd, void *ws, size_t ws_bytes,
                           void *stream, void *const *events);

#ifdef __cplusplus
}
#endif

#endif /* TW_H */
