// sparse_updown.hip -- fused sparse up + down projection over a TwELL gate.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 3-5 equation: for token row m, y_m is the sum over its active
// hidden indices n of (h_g)_{m,n} * (x_m . W_u[:, n]) * W_d[n, :].  Only the
// up column and the down row of an active neuron are read, the up
// activation is a scalar formed in the kernel, and neither h_u nor h is ever
// written to memory.
//
// gfx950 design
// - One workgroup (4 wavefronts) per token row.  The row's tile counts are
//   read once; a row with any tile over capacity is left to the dense
//   backup.  A block-wide scan of the counts gives every packed entry a flat
//   position, and entry f goes to wave f % 4, so the active neurons of a
//   heavy row are shared by four waves.
// - Within a wave, lane l owns the 16-byte chunks l, l+64, ... of a K-row:
//   the gathers of W_u^T[j] and W_d[j] are fully coalesced 1 KB wave loads,
//   x_m stays in registers for the whole row, and y_m accumulates in fp32
//   registers.  Entries are taken two at a time (four row loads in flight
//   per wave): larger batches hold more registers and leave fewer waves
//   resident, which measured slower at every shape (at K = 1024, 78 VGPRs
//   and six waves per SIMD against 112 and four).
// - Batches of at most 256 rows cannot fill the chip with 4 waves per row,
//   and the heaviest row's serial chain of gathers sets the kernel time, so
//   such rows are spread over 16 waves (8 when K > 2048) that take one
//   entry at a time; 32 to 128 rows, over G = 256 / M workgroups, each
//   writing a partial row that row_sum_kernel adds up in a fixed order.
// - Batches of 257 to 8192 rows start their heaviest rows first: a heavy
//   row's chain (176 entries, 22 gathers per wave deep, in the 0.5B block)
//   nearly spans the kernel, so one dispatched late sets its end.  The order
//   (RowOrder in tw_internal.hpp) comes from the extra workgroups of the
//   overflow rows' gate+up launch; workgroup b takes the b-th row of it.
//   Every row is still computed once, by the same code, so y does not depend
//   on the order.
// - The dot product is reduced across the wave with DPP (no LDS), its
//   product with g is the scalar h_j, and h_j * W_d[j] is added lane-wise.
// - The four partial y rows are summed in LDS in a fixed order (the result
//   does not depend on timing) and written once; the staging is laid out so
//   that neither its stores nor its loads have bank conflicts.
// - The overflow rows' dense path runs first.  When its down GEMM split the
//   reduction, workgroup b also sums the partial tiles of overflow-list
//   position b (in split order) into that row of y, so no separate
//   reduction kernel runs: the rows this kernel computes and the overflow
//   rows it finishes are disjoint.
#include "tw_device.hpp"
#include "tw_internal.hpp"
#include "tw_split.hpp"

namespace tw {
namespace {

constexpr int kSmallBatchRows = 256;  // at most this many rows: 16 waves per row

// NWV waves per token row: 4 for large batches; small batches have too few
// rows to fill the chip, and a heavy row's entries then form the critical
// path, so they spread each row over 8 or 16 waves (one entry at a time per
// wave: registers for occupancy rather than loads in flight).
template <int KCH, int NWV>
__global__ __launch_bounds__(NWV * 64) void sparse_updown_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wu_t,
    const uint16_t *__restrict__ wd, int K, int N, int NT, int C,
    const float *__restrict__ tw_val,
    const int32_t *__restrict__ tw_idx, const int32_t *__restrict__ tw_cnt,
    float *__restrict__ y, const float *__restrict__ partial,
    const int32_t *__restrict__ ovf_rows, const int32_t *__restrict__ ovf_count, int R_max,
    int G, float *__restrict__ rowpart, const int32_t *__restrict__ perm) {
    constexpr int kThreads = NWV * 64, kWaves = NWV;
    constexpr int kBatch = NWV >= 8 ? 1 : 2;  // active neurons gathered together per wave
    extern __shared__ __attribute__((aligned(16))) char smem[];  // y staging, fp32
    __shared__ int s_off[kThreads + 1];
    __shared__ int s_wtot[kWaves];

    // G workgroups per row (G = 1: one); part gs of row m
    const int M = gridDim.x / G;
    const int gs = blockIdx.x % G;
    int m = blockIdx.x / G;
    int lead = 0;  // workgroups before the first light row of the order
    if (perm) {
        // heaviest first (G = 1): workgroup b takes the b-th row of "every
        // segment's heavy rows, then every segment's other rows"; lane i
        // scans segment i's two counts
        const int b = blockIdx.x;
        const int nseg = (M + kOrderSeg - 1) / kOrderSeg;
        const int l = threadIdx.x & 63;
        const int nh = l < nseg ? perm[l] : 0, nl = l < nseg ? perm[64 + l] : 0;
        int ih = nh, il = nl;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int vh = __shfl_up(ih, d), vl = __shfl_up(il, d);
            if (l >= d) {
                ih += vh;
                il += vl;
            }
        }
        const int NH = __builtin_amdgcn_readlane(ih, 63);
        lead = NH;
        int sg, idx;
        if (b < NH) {
            sg = (int)__popcll(__ballot(ih <= b));
            idx = b - (__builtin_amdgcn_readlane(ih, sg) - __builtin_amdgcn_readlane(nh, sg));
        } else {
            const int bl = b - NH;
            sg = (int)__popcll(__ballot(il <= bl));
            idx = __builtin_amdgcn_readlane(nh, sg) + bl -
                  (__builtin_amdgcn_readlane(il, sg) - __builtin_amdgcn_readlane(nl, sg));
        }
        // a corrupt order could only come from a corrupt count array: clamp
        sg = min(sg, nseg - 1);
        idx = min(max(idx, 0), kOrderSeg - 1);
        m = (int)min((unsigned)perm[128 + sg * kOrderSeg + idx], (unsigned)(M - 1));
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;

    const int c = tid < NT ? tw_cnt[(size_t)m * NT + tid] : 0;
    if (partial) {
        // overflow-list position p: its split partial tiles, summed in split
        // order into its row of y (S = 1: the down GEMM stored the row).  In
        // the heaviest-first order the duty starts at the first light row
        // (a rotation of the workgroup index, so every position still has
        // exactly one workgroup), off the heavy rows' chains.
        const int p = lead ? (int)(((unsigned)blockIdx.x + (unsigned)(M - lead)) % (unsigned)M)
                           : (int)blockIdx.x;
        const int rows = __builtin_amdgcn_readfirstlane(min(*ovf_count, R_max));
        if (p < rows) {
            const int S = split_factor(rows, K, N);
            if (S > 1) {
                const unsigned row = min((unsigned)ovf_rows[p], (unsigned)(M - 1));
                float *yo = y + (size_t)row * K;
                for (int col = 4 * tid; col < K; col += 4 * kThreads)
                    *reinterpret_cast<float4 *>(yo + col) = split_sum4<8>(partial, p, col, rows, K, S);
            }
        }
    }
    if (__syncthreads_or(c > C)) return;  // overflow row: dense backup

    // exclusive scan of the tile counts -> flat entry offsets
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d);
        if (lane >= d) incl += v;
    }
    if (lane == 63) s_wtot[wave] = incl;
    __syncthreads();
    int wb = 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q)
        if (q < wave) wb += s_wtot[q];
    s_off[tid] = wb + incl - c;
    if (tid == kThreads - 1) s_off[kThreads] = wb + incl;
    __syncthreads();
    const int nnz = s_off[kThreads];

    const int KC = K >> 3;  // 16-byte chunks per K-row
    // this workgroup's output: the row of y, or its partial row
    float *yrow = G > 1 ? rowpart + ((size_t)gs * M + m) * K : y + (size_t)m * K;
    if (nnz == 0) {
        for (int q = tid; q < 2 * KC; q += kThreads)
            st16(yrow + 4 * q, u32x4{0u, 0u, 0u, 0u});
        return;
    }

    u32x4 xr[KCH];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch) {
        const int q = lane + 64 * ch;
        xr[ch] = q < KC ? ld16(x + (size_t)m * K + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    }
    float yacc[KCH][8];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) yacc[ch][e] = 0.0f;

    // entries of this wave: f = gw + GW e, e < ne (gw: the wave's index
    // among the GW = G NWV waves of the row)
    const int gw = gs * kWaves + wave, GW = G * kWaves;
    const int ne = (nnz - gw + GW - 1) / GW;
    for (int e0 = 0; e0 < ne; e0 += 64) {
        // lane resolves entry e0 + lane: tile by binary search over s_off
        int jl = 0;
        float gl = 0.0f;
        if (e0 + lane < ne) {
            const int f = gw + GW * (e0 + lane);
            int lo = 0, hi = NT;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_off[mid] <= f) lo = mid;
                else hi = mid;
            }
            const size_t q = ((size_t)m * NT + lo) * C + (f - s_off[lo]);
            // an index outside [0, N) can only come from a corrupt packing;
            // clamp it so that the gathers stay inside the weights
            jl = min((unsigned)tw_idx[q], (unsigned)(N - 1));
            gl = tw_val[q];
        }
        const int nb = min(64, ne - e0);
        for (int b = 0; b < nb; b += kBatch) {
            int j[kBatch];
            float g[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const bool ok = b + u < nb;
                const int src = ok ? b + u : b;
                j[u] = __builtin_amdgcn_readlane(jl, src);
                g[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), src))
                          : 0.0f;
            }
            u32x4 wu[kBatch][KCH], wv[kBatch][KCH];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const uint16_t *pu = wu_t + (size_t)j[u] * K;
                const uint16_t *pd = wd + (size_t)j[u] * K;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch) {
                    const int q = lane + 64 * ch;
                    const bool in = q < KC;
                    wu[u][ch] = in ? ld16(pu + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                    wv[u][ch] = in ? ld16(pd + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                }
            }
            float p[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                float s = 0.0f;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        s += bf_lo(xr[ch][w]) * bf_lo(wu[u][ch][w]);
                        s += bf_hi(xr[ch][w]) * bf_hi(wu[u][ch][w]);
                    }
                p[u] = s;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) p[u] = wave_sum(p[u]) * g[u];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        yacc[ch][2 * w] += p[u] * bf_lo(wv[u][ch][w]);
                        yacc[ch][2 * w + 1] += p[u] * bf_hi(wv[u][ch][w]);
                    }
        }
    }

    // y staging, transposed: element (ch, e) of lane l of wave w at float
    // ((w KCH + ch) 8 + e) 64 + l, so the 64 lanes of a store hit 64
    // consecutive banks (a lane-contiguous layout, 8 floats per lane, would
    // put 8 lanes on each bank)
    float *s_y = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_y[((wave * KCH + ch) * 8 + e) * 64 + lane] = yacc[ch][e];
    __syncthreads();
    // thread i forms the 4 outputs of half (i / 64) % 2 of lane i % 64's
    // chunk i / 128: consecutive threads read consecutive banks
    for (int i = tid; i < 128 * KCH; i += kThreads) {
        const int l = i & 63, half = (i >> 6) & 1, ch = i >> 7;
        const int q = l + 64 * ch;  // 16-byte chunk of the K-row
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

// y[m] = sum over parts g = 0 .. G-1 (in that order) of the partial rows
// the split sparse kernel wrote, for every row with no tile over capacity
// (the overflow rows hold the dense path's result).
__global__ __launch_bounds__(256) void row_sum_kernel(const float *__restrict__ rowpart, int G,
                                                      int K, int NT, int C,
                                                      const int32_t *__restrict__ tw_cnt,
                                                      float *__restrict__ y) {
    const int m = blockIdx.x, M = gridDim.x, tid = threadIdx.x;
    const int c = tid < NT ? tw_cnt[(size_t)m * NT + tid] : 0;
    if (__syncthreads_or(c > C)) return;
    for (int col = 4 * tid; col < K; col += 4 * 256) {
        float4 v = *reinterpret_cast<const float4 *>(rowpart + (size_t)m * K + col);
        for (int g = 1; g < G; ++g) {
            const float4 u = *reinterpret_cast<const float4 *>(rowpart + ((size_t)g * M + m) * K + col);
            v.x += u.x;
            v.y += u.y;
            v.z += u.z;
            v.w += u.w;
        }
        *reinterpret_cast<float4 *>(y + (size_t)m * K + col) = v;
    }
}

template <int KCH, int NWV>
hipError_t launch_kw(const uint16_t *x, const uint16_t *wu_t, const uint16_t *wd, int M, int K,
                     int N, int NT, int C, const float *tw_val, const int32_t *tw_idx,
                     const int32_t *tw_cnt, float *y, const float *partial,
                     const int32_t *ovf_rows, const int32_t *ovf_count, int R_max, int G,
                     float *rowpart, const int32_t *perm, hipStream_t s) {
    const size_t lds = (size_t)NWV * KCH * 512 * sizeof(float);  // y staging
    {
        const hipError_t e = lds_limit_once<&sparse_updown_kernel<KCH, NWV>>((int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((sparse_updown_kernel<KCH, NWV>), dim3(M * G), dim3(NWV * 64), lds, s, x,
                       wu_t, wd, K, N, NT, C, tw_val, tw_idx, tw_cnt, y, partial, ovf_rows,
                       ovf_count, R_max, G, rowpart, G == 1 ? perm : nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || G == 1) return e;
    hipLaunchKernelGGL(row_sum_kernel, dim3(M), dim3(256), 0, s, rowpart, G, K, NT, C, tw_cnt, y);
    return hipGetLastError();
}

// waves per row by batch size (measured: 16 pays off only while the rows
// alone cannot fill the chip)
template <int KCH>
hipError_t launch_k(const uint16_t *x, const uint16_t *wu_t, const uint16_t *wd, int M, int K,
                    int N, int NT, int C, const float *tw_val, const int32_t *tw_idx,
                    const int32_t *tw_cnt, float *y, const float *partial,
                    const int32_t *ovf_rows, const int32_t *ovf_count, int R_max,
                    float *rowpart, const int32_t *perm, hipStream_t s) {
    // 16 waves cap a lane at 128 registers and the y staging at 16 KCH KB:
    // wide rows take 8
    constexpr int kSmallWaves = KCH <= 4 ? 16 : 8;
    if (M <= kSmallBatchRows)
        return launch_kw<KCH, kSmallWaves>(x, wu_t, wd, M, K, N, NT, C, tw_val, tw_idx, tw_cnt,
                                           y, partial, ovf_rows, ovf_count, R_max,
                                           sparse_row_parts(M), rowpart, perm, s);
    return launch_kw<KCH, 4>(x, wu_t, wd, M, K, N, NT, C, tw_val, tw_idx, tw_cnt, y, partial,
                             ovf_rows, ovf_count, R_max, 1, rowpart, perm, s);
}

}  // namespace

hipError_t launch_sparse_updown(const uint16_t *x, const uint16_t *wu_t, const uint16_t *wd,
                                int M, int K, int N, int T, int C, const float *tw_val,
                                const int32_t *tw_idx, const int32_t *tw_cnt, float *y,
                                const float *partial, const int32_t *ovf_rows,
                                const int32_t *ovf_count, int R_max, float *rowpart,
                                const int32_t *perm, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int NT = N / T;
#define TW_SPARSE_ARGS x, wu_t, wd, M, K, N, NT, C, tw_val, tw_idx, tw_cnt, y, partial, ovf_rows, \
                       ovf_count, R_max, rowpart, perm, s
    switch ((K + 511) / 512) {
    case 1: return launch_k<1>(TW_SPARSE_ARGS);
    case 2: return launch_k<2>(TW_SPARSE_ARGS);
    case 3: return launch_k<3>(TW_SPARSE_ARGS);
    case 4: return launch_k<4>(TW_SPARSE_ARGS);
    case 5: return launch_k<5>(TW_SPARSE_ARGS);
    case 6: return launch_k<6>(TW_SPARSE_ARGS);
    case 7: return launch_k<7>(TW_SPARSE_ARGS);
    default: return launch_k<8>(TW_SPARSE_ARGS);
    }
#undef TW_SPARSE_ARGS
}

}  // namespace tw
