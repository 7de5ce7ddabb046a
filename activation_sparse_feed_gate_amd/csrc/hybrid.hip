// hybrid.hip -- hybrid storage of the gate activation for the training
// forward, and the two products that keep it in that form.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 3-6 (most token rows in a compact ELL-like store of values and
// indices, the few heavy rows whole in a dense backup, a binary routing
// vector per row), section 4-3 (static capacities: at most P stored entries
// per sparse row, a bounded backup, overflow reported for a retry), section
// 2-2 (the training pipeline goes from the TwELL gate to hybrid storage) and
// section 3-7 (dense-to-hybrid and hybrid-to-dense products; in training the
// up and down projections are separate steps that keep the hybrid form).
//
// Kernels
// - hybrid_pack: TwELL -> hybrid.  One wavefront per token row: lane l holds
//   the counts of tiles l, l+64, ...; a wave scan gives each tile's offset
//   in the row's ELL slots, and each lane copies its tiles' entries.  A row
//   whose count exceeds P, or one of whose tiles exceeded the TwELL
//   capacity, is marked in the routing vector instead.
// - route_compact: the ascending list of backup rows from the routing bytes
//   (one workgroup; lane t turns 32 routing bytes into a bit word, then a
//   block scan places the rows), and the true number of backup rows.
// - hybrid_up (sparse rows): u_s = x_m . W_u[:, j_s] for every stored entry,
//   h_s = u_s g_s.  One workgroup of 4 waves per row; entry f goes to wave
//   f % 4; each dot product is a coalesced 1 KB-per-wave gather of the
//   weight row and a DPP wave reduction, four entries in flight per wave.
// - hybrid_down (sparse rows): y_m = sum_s h_s W_d[j_s, :], the down half of
//   the fused inference kernel: the same row split over waves, fp32 partial
//   rows in registers, a fixed-order LDS sum across the 4 waves.
// Backup rows go through the dense MFMA kernels of dense_ffn.hip.
#include "tw_device.hpp"
#include "tw_internal.hpp"
#include "tw_split.hpp"

namespace tw {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ------------------------------- TwELL -> hybrid ---------------------------
__global__ __launch_bounds__(kThreads) void hybrid_pack_kernel(
    const float *__restrict__ tw_val, const int32_t *__restrict__ tw_idx,
    const int32_t *__restrict__ tw_cnt, int M, int NT, int C, int P,
    float *__restrict__ hy_val, int32_t *__restrict__ hy_idx, int32_t *__restrict__ hy_cnt,
    uint8_t *__restrict__ route) {
    const int lane = threadIdx.x & 63;
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (m >= M) return;  // no block barrier below

    constexpr int kQ = 4;  // 64-tile chunks: N / T <= 256
    int c[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int t = lane + 64 * q;
        c[q] = t < NT ? tw_cnt[(size_t)m * NT + t] : 0;
    }
    // exclusive offsets of this lane's tiles in the row, the row total, and
    // whether any tile held more than the TwELL capacity
    int off[kQ], base = 0;
    bool over = false;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        int incl = c[q];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        off[q] = base + incl - c[q];
        base += __shfl(incl, 63);
        over |= c[q] > C;
    }
    const int nnz = base;
    const bool heavy = __any(over) || nnz > P;
    if (lane == 0) {
        hy_cnt[m] = nnz;
        route[m] = heavy ? 1 : 0;
    }
    if (heavy) return;
    // every count is <= C and the offsets stay below nnz <= P
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const size_t src = ((size_t)m * NT + lane + 64 * q) * C;
        const size_t dst = (size_t)m * P + off[q];
        for (int s = 0; s < c[q]; ++s) {
            hy_idx[dst + s] = tw_idx[src + s];
            hy_val[dst + s] = tw_val[src + s];
        }
    }
}

// --------------------------- routing vector -> list ------------------------
__global__ __launch_bounds__(1024) void route_compact_kernel(
    const uint8_t *__restrict__ route, int M, int R_max, int32_t *__restrict__ bk_rows,
    int32_t *__restrict__ bk_count) {
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int running = 0;
    for (int base = 0; base < M; base += 32 * 1024) {
        const int r0 = base + 32 * tid;  // this thread's 32 rows
        uint32_t word = 0;
        if (r0 + 32 <= M) {
            // 16-byte aligned: route is, and r0 is a multiple of 32
            const u32x4 a = ld16(route + r0), b = ld16(route + r0 + 16);
            const uint32_t v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    word |= (((v[i] >> (8 * k)) & 0xffu) ? 1u : 0u) << (4 * i + k);
        } else {
            for (int i = 0; r0 + i < M && i < 32; ++i) word |= (route[r0 + i] ? 1u : 0u) << i;
        }
        const int cnt = __popc(word);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        int wbase = 0, total = 0;
        for (int q = 0; q < 16; ++q) {
            const int v = s_wsum[q];
            if (q < wave) wbase += v;
            total += v;
        }
        int pos = running + wbase + incl - cnt;
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1u;
            if (pos < R_max) bk_rows[pos] = r0 + b;
            ++pos;
        }
        running += total;
        __syncthreads();  // s_wsum is rewritten by the next chunk
    }
    if (tid == 0) *bk_count = running;
}

// ------------------------ dense-to-hybrid products --------------------------
// p_s = a_m . w[j_s] at every stored entry s of a sparse row, then
//   forward  (BWD false): a = x, w = W_u^T:  out1 = p (u, optional), out2 = p g (h)
//   backward (BWD true):  a = dy, w = W_d:   out1 = p g (du), out2 = p u + l1 (dz)
constexpr int kUpBatch = 4;  // entries gathered together per wave

template <int KCH, bool BWD>
__global__ __launch_bounds__(kThreads) void hybrid_up_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wu_t, int K, int N, int P,
    const float *__restrict__ hy_g, const float *__restrict__ hy_uin, float l1,
    const int32_t *__restrict__ hy_idx, const int32_t *__restrict__ hy_cnt,
    const uint8_t *__restrict__ route, float *__restrict__ hy_u, float *__restrict__ hy_h) {
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (route[m]) return;  // backup row: the dense path computes it
    const int n = min(hy_cnt[m], P);
    const int ne = (n - wave + kWaves - 1) / kWaves;  // entries f = wave + 4 e of this wave
    if (ne <= 0) return;

    const int KC = K >> 3;  // 16-byte chunks per K-row
    u32x4 xr[KCH];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch) {
        const int q = lane + 64 * ch;
        xr[ch] = q < KC ? ld16(x + (size_t)m * K + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    }
    const size_t row = (size_t)m * P;
    for (int e0 = 0; e0 < ne; e0 += 64) {
        // lane resolves entry e0 + lane
        const int f = wave + kWaves * (e0 + lane);
        int jl = 0;
        float gl = 0.0f, ul = 0.0f, uin = 0.0f;
        if (e0 + lane < ne) {
            // an index outside [0, N) can only come from corrupt storage;
            // clamp it so that the gather stays inside the weights
            jl = min((unsigned)hy_idx[row + f], (unsigned)(N - 1));
            gl = hy_g[row + f];
            if constexpr (BWD) uin = hy_uin[row + f];
        }
        const int nb = min(64, ne - e0);
        for (int b = 0; b < nb; b += kUpBatch) {
            int j[kUpBatch];
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u)
                j[u] = __builtin_amdgcn_readlane(jl, b + u < nb ? b + u : b);
            u32x4 wu[kUpBatch][KCH];
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u) {
                const uint16_t *pu = wu_t + (size_t)j[u] * K;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch) {
                    const int q = lane + 64 * ch;
                    wu[u][ch] = q < KC ? ld16(pu + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u) {
                float s = 0.0f;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        s += bf_lo(xr[ch][w]) * bf_lo(wu[u][ch][w]);
                        s += bf_hi(xr[ch][w]) * bf_hi(wu[u][ch][w]);
                    }
                s = wave_sum(s);
                if (lane == b + u) ul = s;
            }
        }
        if (e0 + lane < ne) {
            if constexpr (BWD) {
                hy_u[row + f] = ul * gl;
                hy_h[row + f] = ul * uin + l1;
            } else {
                if (hy_u) hy_u[row + f] = ul;
                hy_h[row + f] = ul * gl;
            }
        }
    }
}

// ------------------------- hybrid-to-dense products -------------------------
// out_m = sum over stored s of v1_s w1[j_s] (+ v2_s w2[j_s] with TWO):
//   forward:  v1 = h, w1 = W_d (y);  backward: v1 = du, w1 = W_u^T, v2 = dz,
//   w2 = W_g^T (dx).  TWO gathers two rows per entry, so it takes half as
//   many entries at a time.
template <int KCH, bool TWO>
__global__ __launch_bounds__(kThreads) void hybrid_down_kernel(
    const uint16_t *__restrict__ wd, const uint16_t *__restrict__ w2, int K, int N, int P,
    const float *__restrict__ hy_h, const float *__restrict__ v2,
    const int32_t *__restrict__ hy_idx, const int32_t *__restrict__ hy_cnt,
    const uint8_t *__restrict__ route, float *__restrict__ y, const float *__restrict__ partial,
    const int32_t *__restrict__ bk_rows, const int32_t *__restrict__ bk_count, int R_max,
    int NR) {
    constexpr int kDnBatch = TWO ? 2 : 4;
    extern __shared__ __attribute__((aligned(16))) char smem[];  // y staging, fp32
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (partial) {
        // backup-list position m: the backup GEMM's split partial tiles
        // (reduction depth NR), summed in split order into its row of y
        const int rows = __builtin_amdgcn_readfirstlane(min(*bk_count, R_max));
        if (m < rows) {
            const int S = split_factor(rows, K, NR);
            if (S > 1) {
                const unsigned r = min((unsigned)bk_rows[m], gridDim.x - 1);
                float *yo = y + (size_t)r * K;
                for (int col = 4 * tid; col < K; col += 4 * kThreads)
                    *reinterpret_cast<float4 *>(yo + col) = split_sum4<8>(partial, m, col, rows, K, S);
            }
        }
    }
    if (route[m]) return;  // block-uniform: the backup path writes this row
    const int n = min(hy_cnt[m], P);
    const int KC = K >> 3;
    float *yrow = y + (size_t)m * K;
    if (n == 0) {
        for (int q = tid; q < 2 * KC; q += kThreads) st16(yrow + 4 * q, u32x4{0u, 0u, 0u, 0u});
        return;
    }

    float yacc[KCH][8];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) yacc[ch][e] = 0.0f;

    const size_t row = (size_t)m * P;
    const int ne = (n - wave + kWaves - 1) / kWaves;
    for (int e0 = 0; e0 < ne; e0 += 64) {
        int jl = 0;
        float hl = 0.0f, hl2 = 0.0f;
        if (e0 + lane < ne) {
            const int f = wave + kWaves * (e0 + lane);
            jl = min((unsigned)hy_idx[row + f], (unsigned)(N - 1));
            hl = hy_h[row + f];
            if constexpr (TWO) hl2 = v2[row + f];
        }
        const int nb = min(64, ne - e0);
        for (int b = 0; b < nb; b += kDnBatch) {
            int j[kDnBatch];
            float h[kDnBatch], h2[kDnBatch];
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                const bool ok = b + u < nb;
                const int src = ok ? b + u : b;
                j[u] = __builtin_amdgcn_readlane(jl, src);
                h[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl), src))
                          : 0.0f;
                h2[u] = ok && TWO
                            ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl2), src))
                            : 0.0f;
            }
            u32x4 wv[kDnBatch][KCH], wv2[TWO ? kDnBatch : 1][KCH];
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                const uint16_t *pd = wd + (size_t)j[u] * K;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch) {
                    const int q = lane + 64 * ch;
                    wv[u][ch] = q < KC ? ld16(pd + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                }
                if constexpr (TWO) {
                    const uint16_t *p2 = w2 + (size_t)j[u] * K;
#pragma unroll
                    for (int ch = 0; ch < KCH; ++ch) {
                        const int q = lane + 64 * ch;
                        wv2[u][ch] = q < KC ? ld16(p2 + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u)
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        yacc[ch][2 * w] += h[u] * bf_lo(wv[u][ch][w]);
                        yacc[ch][2 * w + 1] += h[u] * bf_hi(wv[u][ch][w]);
                        if constexpr (TWO) {
                            yacc[ch][2 * w] += h2[u] * bf_lo(wv2[u][ch][w]);
                            yacc[ch][2 * w + 1] += h2[u] * bf_hi(wv2[u][ch][w]);
                        }
                    }
        }
    }

    // y staging, transposed as in the fused inference kernel: element
    // (ch, e) of lane l of wave w at float ((w KCH + ch) 8 + e) 64 + l, so
    // neither the stores nor the loads below have bank conflicts
    float *s_y = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_y[((wave * KCH + ch) * 8 + e) * 64 + lane] = yacc[ch][e];
    __syncthreads();
    for (int i = tid; i < 128 * KCH; i += kThreads) {
        const int l = i & 63, half = (i >> 6) & 1, ch = i >> 7;
        const int q = l + 64 * ch;
        if (q >= KC) continue;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = (ch * 8 + 4 * half + e) * 64 + l;
            float v = s_y[o];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) v += s_y[(size_t)w * KCH * 512 + o];
            r[e] = v;
        }
        st16(yrow + 8 * q + 4 * half, u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]),
                                            __float_as_uint(r[2]), __float_as_uint(r[3])});
    }
}

// ------------------------------ hybrid transpose ----------------------------
// Column lists of the sparse rows' stored entries (id = m P + s), for the
// weight gradients: grouped by hidden column j and, within a column, in
// ascending row order (so the gradient sums have a fixed order).  Counts
// (atomic, order free), an exclusive scan to column offsets, a scatter
// through per-column cursors (order within a column depends on timing), then
// a per-column rank sort by row (a row appears at most once in a column).
// The backup rows' contributions are dense products on the matrix cores.
__global__ __launch_bounds__(kThreads) void fill_i32_kernel(int32_t *__restrict__ p, int n,
                                                             int32_t v) {
    for (int i = blockIdx.x * kThreads + threadIdx.x; i < n; i += gridDim.x * kThreads) p[i] = v;
}

// SCATTER false: count entries per column; true: place (row, id) through the
// cursors.  One wave per sparse row.
template <bool SCATTER>
__global__ __launch_bounds__(kThreads) void tr_place_kernel(
    int M, int N, int P, const int32_t *__restrict__ hy_idx, const int32_t *__restrict__ hy_cnt,
    const uint8_t *__restrict__ route, int32_t *__restrict__ col, int32_t *__restrict__ ent_row,
    int32_t *__restrict__ ent_id) {
    const int lane = threadIdx.x & 63;
    const int m = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (m >= M || route[m]) return;
    const int n = min(hy_cnt[m], P);
    for (int s = lane; s < n; s += 64) {
        const int j = min((unsigned)hy_idx[(size_t)m * P + s], (unsigned)(N - 1));
        if constexpr (SCATTER) {
            const int pos = atomicAdd(&col[j], 1);
            ent_row[pos] = m;
            ent_id[pos] = m * P + s;
        } else {
            atomicAdd(&col[j], 1);
        }
    }
}

// col_ptr = exclusive scan of the counts (col_ptr[N] = total); the counts
// become the scatter cursors (each column's start).
__global__ __launch_bounds__(1024) void tr_scan_kernel(int32_t *__restrict__ col, int N,
                                                       int32_t *__restrict__ col_ptr) {
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int running = 0;
    for (int base = 0; base < N; base += 1024) {
        const int j = base + tid;
        const int c = j < N ? col[j] : 0;
        int incl = c;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        int wbase = 0, total = 0;
        for (int q = 0; q < 16; ++q) {
            const int v = s_wsum[q];
            if (q < wave) wbase += v;
            total += v;
        }
        if (j < N) {
            const int start = running + wbase + incl - c;
            col_ptr[j] = start;
            col[j] = start;
        }
        running += total;
        __syncthreads();
    }
    if (tid == 0) col_ptr[N] = running;
}

// One wave per column: the rank of an entry is the number of the column's
// entries with a smaller row; 64 keys at a time are held in a register and
// compared through lane reads.
__global__ __launch_bounds__(kThreads) void tr_sort_kernel(
    int N, const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ ent_row,
    const int32_t *__restrict__ ent_id, int32_t *__restrict__ srt_row,
    int32_t *__restrict__ srt_id) {
    const int j = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (j >= N) return;
    const int lane = threadIdx.x & 63;
    const int p0 = col_ptr[j], n = col_ptr[j + 1] - p0;
    for (int c = 0; c < n; c += 64) {
        const int i = c + lane;
        const int my = i < n ? ent_row[p0 + i] : 0x7fffffff;
        int rank = 0;
        for (int c2 = 0; c2 < n; c2 += 64) {
            const int key = c2 + lane < n ? ent_row[p0 + c2 + lane] : 0x7fffffff;
            const int nk = min(64, n - c2);
            for (int t = 0; t < nk; ++t) rank += __builtin_amdgcn_readlane(key, t) < my ? 1 : 0;
        }
        if (i < n) {
            srt_row[p0 + rank] = my;
            srt_id[p0 + rank] = ent_id[p0 + i];
        }
    }
}

// --------------------------- weight gradients --------------------------------
// One wave per hidden column j (and K-slice of up to KS 16-byte chunks per
// lane): over the column's entries in ascending row order,
//   dwd[j] = sum h dy_m,   dwu_t[j] = sum du x_m,   dwg_t[j] = sum dz x_m
// gathering the dy and x rows (bf16, coalesced 1 KB per wave and chunk) with
// the sparse rows' fp32 values.  fp32 accumulation; every output row is
// written (zeros for columns with no entry).
constexpr int kDwBatch = 2;

template <int KS>
__global__ __launch_bounds__(kThreads) void dw_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dy, int M, int K, int N, int P,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ srt_row,
    const int32_t *__restrict__ srt_id, const float *__restrict__ hy_h,
    const float *__restrict__ hy_du, const float *__restrict__ hy_dz, float *__restrict__ dwg_t,
    float *__restrict__ dwu_t, float *__restrict__ dwd) {
    const int j = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
    if (j >= N) return;
    const int lane = threadIdx.x & 63;
    const int KC = K >> 3;
    const int q0 = blockIdx.y * KS * 64;  // first chunk of this K-slice
    const int MP = M * P;
    float ad[KS][8], au[KS][8], ag[KS][8];
#pragma unroll
    for (int c = 0; c < KS; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) ad[c][e] = au[c][e] = ag[c][e] = 0.0f;

    const int p0 = col_ptr[j], n = col_ptr[j + 1] - p0;
    for (int e0 = 0; e0 < n; e0 += 64) {
        int ml = 0;
        float hl = 0.0f, ul = 0.0f, zl = 0.0f;
        if (e0 + lane < n) {
            ml = min((unsigned)srt_row[p0 + e0 + lane], (unsigned)(M - 1));
            const int id = min((unsigned)srt_id[p0 + e0 + lane], (unsigned)(MP - 1));
            hl = hy_h[id];
            ul = hy_du[id];
            zl = hy_dz[id];
        }
        const int nb = min(64, n - e0);
        for (int b = 0; b < nb; b += kDwBatch) {
            int m[kDwBatch];
            float h[kDwBatch], du[kDwBatch], dz[kDwBatch];
#pragma unroll
            for (int u = 0; u < kDwBatch; ++u) {
                const bool ok = b + u < nb;
                const int src = ok ? b + u : b;
                m[u] = __builtin_amdgcn_readlane(ml, src);
                h[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl), src)) : 0.0f;
                du[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ul), src)) : 0.0f;
                dz[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(zl), src)) : 0.0f;
            }
            u32x4 gy[kDwBatch][KS], gx[kDwBatch][KS];
#pragma unroll
            for (int u = 0; u < kDwBatch; ++u)
#pragma unroll
                for (int c = 0; c < KS; ++c) {
                    const int q = q0 + lane + 64 * c;
                    const bool in = q < KC;
                    gy[u][c] = in ? ld16(dy + (size_t)m[u] * K + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                    gx[u][c] = in ? ld16(x + (size_t)m[u] * K + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                }
#pragma unroll
            for (int u = 0; u < kDwBatch; ++u)
#pragma unroll
                for (int c = 0; c < KS; ++c)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        ad[c][2 * w] += h[u] * bf_lo(gy[u][c][w]);
                        ad[c][2 * w + 1] += h[u] * bf_hi(gy[u][c][w]);
                        au[c][2 * w] += du[u] * bf_lo(gx[u][c][w]);
                        au[c][2 * w + 1] += du[u] * bf_hi(gx[u][c][w]);
                        ag[c][2 * w] += dz[u] * bf_lo(gx[u][c][w]);
                        ag[c][2 * w + 1] += dz[u] * bf_hi(gx[u][c][w]);
                    }
        }
    }
#pragma unroll
    for (int c = 0; c < KS; ++c) {
        const int q = q0 + lane + 64 * c;
        if (q >= KC) continue;
        const size_t o = (size_t)j * K + 8 * q;
        float *outs[3] = {dwd + o, dwu_t + o, dwg_t + o};
        const float(*acc[3])[8] = {ad, au, ag};
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            st16(outs[t], u32x4{__float_as_uint(acc[t][c][0]), __float_as_uint(acc[t][c][1]),
                                __float_as_uint(acc[t][c][2]), __float_as_uint(acc[t][c][3])});
            st16(outs[t] + 4, u32x4{__float_as_uint(acc[t][c][4]), __float_as_uint(acc[t][c][5]),
                                    __float_as_uint(acc[t][c][6]), __float_as_uint(acc[t][c][7])});
        }
    }
}

template <int KCH, bool BWD>
hipError_t launch_up_k(const uint16_t *x, const uint16_t *wu_t, int M, int K, int N, int P,
                       const float *hy_g, const float *hy_uin, float l1, const int32_t *hy_idx,
                       const int32_t *hy_cnt, const uint8_t *route, float *hy_u, float *hy_h,
                       hipStream_t s) {
    hipLaunchKernelGGL((hybrid_up_kernel<KCH, BWD>), dim3(M), dim3(kThreads), 0, s, x, wu_t, K,
                       N, P, hy_g, hy_uin, l1, hy_idx, hy_cnt, route, hy_u, hy_h);
    return hipGetLastError();
}

template <int KCH, bool TWO>
hipError_t launch_down_k(const uint16_t *wd, const uint16_t *w2, int M, int K, int N, int P,
                         const float *hy_h, const float *v2, const int32_t *hy_idx,
                         const int32_t *hy_cnt, const uint8_t *route, float *y,
                         const float *partial, const int32_t *bk_rows, const int32_t *bk_count,
                         int R_max, hipStream_t s) {
    const size_t lds = (size_t)kWaves * KCH * 512 * sizeof(float);
    {
        const hipError_t e = lds_limit_once<&hybrid_down_kernel<KCH, TWO>>((int)lds);
        if (e != hipSuccess) return e;
    }
    // the backup GEMM's reduction: N deep, or 2 N for the two products of dx
    hipLaunchKernelGGL((hybrid_down_kernel<KCH, TWO>), dim3(M), dim3(kThreads), lds, s, wd, w2,
                       K, N, P, hy_h, v2, hy_idx, hy_cnt, route, y, partial, bk_rows, bk_count,
                       R_max, TWO ? 2 * N : N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hybrid_pack(const float *tw_val, const int32_t *tw_idx, const int32_t *tw_cnt,
                              int M, int N, int T, int C, int P, float *hy_val, int32_t *hy_idx,
                              int32_t *hy_cnt, uint8_t *route, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(hybrid_pack_kernel, dim3((M + kWaves - 1) / kWaves), dim3(kThreads), 0, s,
                       tw_val, tw_idx, tw_cnt, M, N / T, C, P, hy_val, hy_idx, hy_cnt, route);
    return hipGetLastError();
}

hipError_t launch_route_compact(const uint8_t *route, int M, int R_max, int32_t *bk_rows,
                                int32_t *bk_count, hipStream_t s) {
    hipLaunchKernelGGL(route_compact_kernel, dim3(1), dim3(1024), 0, s, route, M, R_max, bk_rows,
                       bk_count);
    return hipGetLastError();
}

#define TW_KCH_SWITCH(K, CALL)            \
    switch (((K) + 511) / 512) {          \
    case 1: return CALL(1);               \
    case 2: return CALL(2);               \
    case 3: return CALL(3);               \
    case 4: return CALL(4);               \
    case 5: return CALL(5);               \
    case 6: return CALL(6);               \
    case 7: return CALL(7);               \
    default: return CALL(8);              \
    }

hipError_t launch_hybrid_up(const uint16_t *x, const uint16_t *wu_t, int M, int K, int N, int P,
                            const float *hy_g, const int32_t *hy_idx, const int32_t *hy_cnt,
                            const uint8_t *route, float *hy_u, float *hy_h, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define TW_UP(k) \
    launch_up_k<k, false>(x, wu_t, M, K, N, P, hy_g, nullptr, 0.0f, hy_idx, hy_cnt, route, hy_u, \
                          hy_h, s)
    TW_KCH_SWITCH(K, TW_UP)
#undef TW_UP
}

hipError_t launch_hybrid_dh(const uint16_t *dy, const uint16_t *wd, int M, int K, int N, int P,
                            const float *hy_g, const float *hy_u, float l1, const int32_t *hy_idx,
                            const int32_t *hy_cnt, const uint8_t *route, float *hy_du,
                            float *hy_dz, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define TW_DH(k) \
    launch_up_k<k, true>(dy, wd, M, K, N, P, hy_g, hy_u, l1, hy_idx, hy_cnt, route, hy_du, \
                         hy_dz, s)
    TW_KCH_SWITCH(K, TW_DH)
#undef TW_DH
}

hipError_t launch_hybrid_down(const uint16_t *wd, int M, int K, int N, int P, const float *hy_h,
                              const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                              float *y, const float *partial, const int32_t *bk_rows,
                              const int32_t *bk_count, int R_max, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define TW_DN(k) \
    launch_down_k<k, false>(wd, nullptr, M, K, N, P, hy_h, nullptr, hy_idx, hy_cnt, route, y, \
                            partial, bk_rows, bk_count, R_max, s)
    TW_KCH_SWITCH(K, TW_DN)
#undef TW_DN
}

hipError_t launch_hybrid_dx(const uint16_t *wu_t, const uint16_t *wg_t, int M, int K, int N,
                            int P, const float *hy_du, const float *hy_dz,
                            const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                            float *dx, const float *partial, const int32_t *bk_rows,
                            const int32_t *bk_count, int R_max, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define TW_DX(k) \
    launch_down_k<k, true>(wu_t, wg_t, M, K, N, P, hy_du, hy_dz, hy_idx, hy_cnt, route, dx, \
                           partial, bk_rows, bk_count, R_max, s)
    TW_KCH_SWITCH(K, TW_DX)
#undef TW_DX
}

// workspace of launch_hybrid_dw: column counts / cursors, column offsets,
// the scattered and the sorted (row, id) lists of the M P stored slots, then
// the backup rows' gathered dy and x (32-row padded)
size_t hybrid_dw_bytes(int M, int K, int N, int P, int R_max) {
    const size_t cap = (size_t)M * P;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    return up((size_t)N * 4) + up((size_t)(N + 1) * 4) + 4 * up(cap * 4) +
           2 * up(backup_gather_bytes(R_max, K));
}

hipError_t launch_hybrid_dw(const uint16_t *x, const uint16_t *dy, int M, int K, int N, int P,
                            const float *hy_h, const float *hy_du, const float *hy_dz,
                            const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                            const int32_t *bk_rows, const int32_t *bk_count, int R_max,
                            const uint16_t *bk_h, const uint16_t *bk_du, const uint16_t *bk_dz,
                            float *dwg_t, float *dwu_t, float *dwd, void *ws, hipStream_t s,
                            hipEvent_t ev_transposed, hipEvent_t ev_sparse) {
    const size_t cap = (size_t)M * P;
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    char *w = static_cast<char *>(ws);
    int32_t *col = reinterpret_cast<int32_t *>(w);
    w += up((size_t)N * 4);
    int32_t *col_ptr = reinterpret_cast<int32_t *>(w);
    w += up((size_t)(N + 1) * 4);
    int32_t *ent_row = reinterpret_cast<int32_t *>(w);
    w += up(cap * 4);
    int32_t *ent_id = reinterpret_cast<int32_t *>(w);
    w += up(cap * 4);
    int32_t *srt_row = reinterpret_cast<int32_t *>(w);
    w += up(cap * 4);
    int32_t *srt_id = reinterpret_cast<int32_t *>(w);
    w += up(cap * 4);
    uint16_t *dy_bk = reinterpret_cast<uint16_t *>(w);
    w += up(backup_gather_bytes(R_max, K));
    uint16_t *x_bk = reinterpret_cast<uint16_t *>(w);

    const int fill_grid = (N + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(fill_i32_kernel, dim3(fill_grid < 1024 ? fill_grid : 1024), dim3(kThreads),
                       0, s, col, N, 0);
    const int place_grid = (M + kWaves - 1) / kWaves;
    if (place_grid > 0)
        hipLaunchKernelGGL(tr_place_kernel<false>, dim3(place_grid), dim3(kThreads), 0, s, M, N,
                           P, hy_idx, hy_cnt, route, col, ent_row, ent_id);
    hipLaunchKernelGGL(tr_scan_kernel, dim3(1), dim3(1024), 0, s, col, N, col_ptr);
    if (place_grid > 0)
        hipLaunchKernelGGL(tr_place_kernel<true>, dim3(place_grid), dim3(kThreads), 0, s, M, N, P,
                           hy_idx, hy_cnt, route, col, ent_row, ent_id);
    const int cgrid = (N + kWaves - 1) / kWaves;
    hipLaunchKernelGGL(tr_sort_kernel, dim3(cgrid), dim3(kThreads), 0, s, N, col_ptr, ent_row,
                       ent_id, srt_row, srt_id);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev_transposed && (e = hipEventRecord(ev_transposed, s)) != hipSuccess) return e;
    const int KCH = (K + 511) / 512;
#define TW_DW(ks, slices)                                                                        \
    hipLaunchKernelGGL(dw_kernel<ks>, dim3(cgrid, slices), dim3(kThreads), 0, s, x, dy, M, K, N, \
                       P, col_ptr, srt_row, srt_id, hy_h, hy_du, hy_dz, dwg_t, dwu_t, dwd)
    switch (KCH) {
    case 1: TW_DW(1, 1); break;
    case 2: TW_DW(2, 1); break;
    case 3: TW_DW(3, 1); break;
    default: TW_DW(4, (KCH + 3) / 4); break;
    }
#undef TW_DW
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev_sparse && (e = hipEventRecord(ev_sparse, s)) != hipSuccess) return e;
    // the backup rows: dW += T^T G on the matrix cores
    return launch_backup_wgrad(dy, x, K, N, bk_rows, bk_count, R_max, bk_h, bk_du, bk_dz, dy_bk,
                               x_bk, dwd, dwu_t, dwg_t, s);
}

}  // namespace tw
