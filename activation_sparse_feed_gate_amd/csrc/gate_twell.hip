// gate_twell.hip -- gate GEMM with a ReLU + TwELL-packing epilogue, and the
// compaction of the rows that overflow a tile's capacity.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 3-4 (TwELL, and the five-step fused gate kernel: load tiles, matrix
// multiply, ReLU, local count and pack, write the packed form instead of the
// dense gate), section 3-6 and 4-3 (rows over capacity are routed whole to a
// dense backup through a routing vector; overflow beyond the backup room is
// reported for a retry).
//
// gfx950 design
// - Macro tile 256 rows x 256 columns, 4 waves in a 2 x 2 grid, each wave
//   owning 128 x 128 outputs as 4 x 4 blocks of v_mfma_f32_32x32x16_bf16
//   (256 fp32 accumulators per lane).  K advances 64 at a time through a
//   double-buffered, XOR-swizzled LDS stage (2 x 64 KB).
// - Epilogue without an LDS round trip: in the 32x32 MFMA result layout one
//   accumulator register of a block holds 32 consecutive columns of two rows
//   (lanes 0-31 and 32-63), so one 64-bit wavefront ballot of (z > 0) gives
//   the activity masks of both rows.  Popcounts of the masks give the counts,
//   and popcount of the mask bits below a lane gives its slot, in ascending
//   column order.  With T = 128 a tile is exactly one wave's 128 columns;
//   with T = 256 it spans the two waves of a wave row, which exchange their
//   half counts through LDS.
// - Each workgroup writes one bit per row (overflowing or not) for its column
//   block, so no buffer needs clearing beforehand; the compaction kernel ORs
//   the column blocks and lists the set rows in ascending order.
#include "tw_device.hpp"
#include "tw_internal.hpp"

namespace tw {
namespace {

constexpr int kThreads = 256;
constexpr int kStageBytes = kGateBM * kRowBytes;           // 32 KB per operand
constexpr int kLdsTiles = 4 * kStageBytes;                  // A, B double-buffered
constexpr int kLdsBytes = kLdsTiles + 64 + 2 * kGateBM * 4; // + row flags + half counts

template <int T>
__global__ __launch_bounds__(kThreads) void gate_twell_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg_t, int M, int K, int N,
    int C, int NBN, float *__restrict__ tw_val, int32_t *__restrict__ tw_idx,
    int32_t *__restrict__ tw_cnt, uint32_t *__restrict__ oflag, float *__restrict__ zdbg) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    char *As = smem;
    char *Bs = smem + 2 * kStageBytes;
    uint32_t *s_flag = reinterpret_cast<uint32_t *>(smem + kLdsTiles);
    int *s_half = reinterpret_cast<int *>(smem + kLdsTiles + 64);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int bn = blockIdx.x % NBN;
    const int bm = blockIdx.x / NBN;
    const int m0 = bm * kGateBM, n0 = bn * kGateBN;

    if (tid < 8) s_flag[tid] = 0u;

    // This thread moves chunk kc = tid % 8 of tile rows tid/8 + 32*i, i < 8.
    const int r0 = tid >> 3, kc0 = tid & 7;
    int aoff[8], boff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int ra = min(m0 + r0 + 32 * i, M - 1);
        const int rb = min(n0 + r0 + 32 * i, N - 1);
        aoff[i] = ra * K + kc0 * 8;
        boff[i] = rb * K + kc0 * 8;
    }
    u32x4 ra[8], rb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ra[i] = ld16(x + aoff[i]);
        rb[i] = ld16(wg_t + boff[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        lds_st16(As, lds_off(r0 + 32 * i, kc0), ra[i]);
        lds_st16(Bs, lds_off(r0 + 32 * i, kc0), rb[i]);
    }
    __syncthreads();

    f32x16 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    const int KT = K / kBK;
    const int frow = lane & 31;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) {
            const int k1 = (kt + 1) * kBK;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                ra[i] = ld16(x + aoff[i] + k1);
                rb[i] = ld16(wg_t + boff[i] + k1);
            }
        }
        const char *Ac = As + cur * kStageBytes;
        const char *Bc = Bs + cur * kStageBytes;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int kc = 2 * s + (lane >> 5);
            u32x4 fa[4], fb[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) fa[a] = lds_ld16(Ac, lds_off(wm * 128 + a * 32 + frow, kc));
#pragma unroll
            for (int b = 0; b < 4; ++b) fb[b] = lds_ld16(Bc, lds_off(wn * 128 + b * 32 + frow, kc));
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(fa[a], fb[b], acc[a][b]);
        }
        if (more) {
            char *An = As + (cur ^ 1) * kStageBytes;
            char *Bn = Bs + (cur ^ 1) * kStageBytes;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                lds_st16(An, lds_off(r0 + 32 * i, kc0), ra[i]);
                lds_st16(Bn, lds_off(r0 + 32 * i, kc0), rb[i]);
            }
        }
        __syncthreads();
    }

    // ---------------- epilogue: ReLU + TwELL pack + row overflow bits ----
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const uint32_t below = (1u << l32) - 1u;
    const int ncol0 = n0 + wn * 128;  // first column of this wave
    const bool live = ncol0 < N;      // false only in a half-empty last column block
    const int NT = N / T;
    const int t = ncol0 / T;

    if (T == 256) {
        // pass 1: this wave's half-tile count of every row it holds
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int tot = 0;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint64_t bal = __ballot(acc[a][b][i] > 0.0f);
                    tot += __popc(half ? (uint32_t)(bal >> 32) : (uint32_t)bal);
                }
                const int rloc = wm * 128 + a * 32 + mfma32_row(i, lane);
                if (l32 == 0) s_half[wn * kGateBM + rloc] = tot;
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rloc = wm * 128 + a * 32 + mfma32_row(i, lane);
            const int m = m0 + rloc;
            uint32_t mk[4];
            int pre[4];
            int tot = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint64_t bal = __ballot(acc[a][b][i] > 0.0f);
                mk[b] = half ? (uint32_t)(bal >> 32) : (uint32_t)bal;
                pre[b] = tot;
                tot += __popc(mk[b]);
            }
            int off = 0, total = tot;
            bool owner = true;  // the wave that stores the count of this (row, tile)
            if (T == 256) {
                const int other = s_half[(wn ^ 1) * kGateBM + rloc];
                off = wn ? other : 0;
                total = tot + other;
                owner = wn == 0;
            }
            if (m < M && live) {
                const size_t tb = ((size_t)m * NT + t) * C;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const float v = acc[a][b][i];
                    if (v > 0.0f) {
                        const int slot = off + pre[b] + __popc(mk[b] & below);
                        if (slot < C) {
                            tw_idx[tb + slot] = ncol0 + b * 32 + l32;
                            tw_val[tb + slot] = v;
                        }
                    }
                }
                if (owner && l32 == 0) {
                    tw_cnt[(size_t)m * NT + t] = total;
                    if (total > C) atomicOr(&s_flag[rloc >> 5], 1u << (rloc & 31));
                }
                if (zdbg) {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        zdbg[(size_t)m * N + ncol0 + b * 32 + l32] = acc[a][b][i];
                }
            }
        }
    }
    __syncthreads();
    const int MW = (M + 31) >> 5;
    if (tid < 8 && m0 + 32 * tid < M) oflag[(size_t)bn * MW + (m0 >> 5) + tid] = s_flag[tid];
}

// Ascending list of the rows whose bit is set in any column block.  One
// workgroup: each thread ORs one 32-row word over the column blocks, a
// block-wide scan of the popcounts gives every set bit its list position.
__global__ __launch_bounds__(1024) void ovf_compact_kernel(const uint32_t *__restrict__ oflag,
                                                           int NB, int MW, int R_max,
                                                           int32_t *__restrict__ ovf_rows,
                                                           int32_t *__restrict__ ovf_count) {
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int running = 0;
    for (int base = 0; base < MW; base += 1024) {
        const int w = base + tid;
        uint32_t word = 0;
        if (w < MW)
            for (int nb = 0; nb < NB; ++nb) word |= oflag[(size_t)nb * MW + w];
        const int c = __popc(word);
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
        int pos = running + wbase + incl - c;
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1u;
            if (pos < R_max) ovf_rows[pos] = w * 32 + b;
            ++pos;
        }
        running += total;
        __syncthreads();
    }
    if (tid == 0) *ovf_count = running;
}

template <int T>
hipError_t launch_gate_t(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N, int C,
                         float *tw_val, int32_t *tw_idx, int32_t *tw_cnt, uint32_t *oflag,
                         float *z_debug, hipStream_t s) {
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gate_twell_kernel<T>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int NBN = gate_col_blocks(N);
    const int NBM = (M + kGateBM - 1) / kGateBM;
    hipLaunchKernelGGL(gate_twell_kernel<T>, dim3(NBN * NBM), dim3(kThreads), kLdsBytes, s, x,
                       wg_t, M, K, N, C, NBN, tw_val, tw_idx, tw_cnt, oflag, z_debug);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_twell(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N,
                             int T, int C, float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                             uint32_t *oflag, float *z_debug, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (T == 128)
        return launch_gate_t<128>(x, wg_t, M, K, N, C, tw_val, tw_idx, tw_cnt, oflag, z_debug, s);
    return launch_gate_t<256>(x, wg_t, M, K, N, C, tw_val, tw_idx, tw_cnt, oflag, z_debug, s);
}

hipError_t launch_ovf_compact(const uint32_t *oflag, int NB, int MW, int R_max,
                              int32_t *ovf_rows, int32_t *ovf_count, hipStream_t s) {
    hipLaunchKernelGGL(ovf_compact_kernel, dim3(1), dim3(1024), 0, s, oflag, NB, MW, R_max,
                       ovf_rows, ovf_count);
    return hipGetLastError();
}

}  // namespace tw
