// pack_dense.hip -- TwELL packing and overflow routing of a dense gate
// matrix already in memory: the second half of the unfused baseline that
// the fused gate kernel is measured against, and a packer for gates that
// were computed elsewhere.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 3-4 (TwELL: per row and column tile, the active values, their
// original indices and the true count; packing in the gate's epilogue
// instead of a separate pass that writes, reads and writes again) and
// sections 3-6 / 4-3 (rows over capacity are routed to the dense backup).
//
// gfx950 design
// - One workgroup (4 waves) per block of 32 rows x 256 columns, the
//   granularity of one row-overflow word of the compaction: wave w packs
//   rows 8w .. 8w+7 of the block and issues all eight 1 KB row loads before
//   the first one is used.
// - Lane l holds columns 4l .. 4l+3 of the block.  With T = 128, lanes 0-31
//   and 32-63 are two tiles; with T = 256 all 64 lanes are one tile.  The
//   lane's active count, an inclusive scan over the lanes of its tile and
//   the tile's total give every active entry its slot in ascending column
//   order, exactly as the fused epilogue does.
#include "tw_device.hpp"
#include "tw_internal.hpp"

namespace tw {
namespace {

template <int T>
__global__ __launch_bounds__(256) void pack_dense_kernel(
    const float *__restrict__ z, int M, int N, int C, int MW, float *__restrict__ tw_val,
    int32_t *__restrict__ tw_idx, int32_t *__restrict__ tw_cnt, uint32_t *__restrict__ oflag) {
    constexpr int G = T / 4;  // lanes per tile
    __shared__ uint32_t s_word;
    const int w = blockIdx.x % MW, nb = blockIdx.x / MW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NT = N / T;
    const int c0 = nb * 256 + 4 * lane;  // first column of this lane
    const bool colok = c0 < N;           // N is a multiple of 128: whole lanes in or out
    const int t = (nb * 256 + 4 * (lane & ~(G - 1))) / T;
    const int gl = lane & (G - 1);       // lane within its tile
    if (tid == 0) s_word = 0u;

    float4 v[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int m = 32 * w + 8 * wave + r;
        v[r] = (m < M && colok) ? *reinterpret_cast<const float4 *>(z + (size_t)m * N + c0)
                                : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    __syncthreads();  // s_word is cleared

    uint32_t over = 0;  // bit 8 wave + r: that row has a tile over capacity (wave-uniform)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int m = 32 * w + 8 * wave + r;
        const float e[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) bits |= (e[k] > 0.0f ? 1u : 0u) << k;
        const int cnt = __popc(bits);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < G; d <<= 1) {
            const int u = __shfl_up(incl, d);
            if (gl >= d) incl += u;
        }
        const int total = __shfl(incl, (lane & ~(G - 1)) + G - 1);  // the tile's count
        if (m < M && colok) {
            const size_t tb = ((size_t)m * NT + t) * C;
            int slot = incl - cnt;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if ((bits >> k) & 1u) {
                    if (slot < C) {
                        tw_idx[tb + slot] = c0 + k;
                        tw_val[tb + slot] = e[k];
                    }
                    ++slot;
                }
            if (gl == 0) tw_cnt[(size_t)m * NT + t] = total;
        }
        if (__ballot(gl == 0 && colok && m < M && total > C)) over |= 1u << (8 * wave + r);
    }
    if (lane == 0 && over) atomicOr(&s_word, over);
    __syncthreads();
    if (tid == 0) oflag[(size_t)nb * MW + w] = s_word;
}

}  // namespace

hipError_t launch_pack_dense(const float *z, int M, int N, int T, int C, float *tw_val,
                             int32_t *tw_idx, int32_t *tw_cnt, uint32_t *oflag, hipStream_t s) {
    if (M == 0) return hipSuccess;
    const int MW = row_words(M);
    const int grid = gate_col_blocks(N) * MW;
    if (T == 128)
        hipLaunchKernelGGL(pack_dense_kernel<128>, dim3(grid), dim3(256), 0, s, z, M, N, C, MW,
                           tw_val, tw_idx, tw_cnt, oflag);
    else
        hipLaunchKernelGGL(pack_dense_kernel<256>, dim3(grid), dim3(256), 0, s, z, M, N, C, MW,
                           tw_val, tw_idx, tw_cnt, oflag);
    return hipGetLastError();
}

}  // namespace tw
