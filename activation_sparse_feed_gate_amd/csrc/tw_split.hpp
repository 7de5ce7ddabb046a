// tw_split.hpp -- the split reduction of the row-list down GEMM: how many
// splits it takes and where it leaves its partial tiles.  The GEMM, the
// kernel that sums the partials and the sparse kernel (which sums the
// overflow rows' partials beside its own rows) all evaluate these from the
// same device-side row count.
#pragma once

#include "tw_gemm.hpp"

namespace tw {

constexpr int kSplitGrid = 256;  // work items (workgroups) of the split down GEMM
constexpr int kSplitBM = 128;    // its output tile: listed rows
constexpr int kSplitBN = 128;    // and output columns

// Reduction splits for `tiles` output tiles and `grid` work items: enough to
// occupy the grid, at most 16, dividing the NS stages of the reduction.
__device__ __forceinline__ int split_count(int tiles, int grid, int NS) {
    if (tiles <= 0) return 1;
    int S = grid / tiles;
    S = S < 1 ? 1 : (S > 16 ? 16 : S);
    while (NS % S) --S;
    return S;
}

// Splits of the row-list down GEMM over `rows` listed rows, output width K
// and reduction depth N (1: it stored its rows itself).
__device__ __forceinline__ int split_factor(int rows, int K, int N) {
    const int nrb = (rows + kSplitBM - 1) / kSplitBM;
    return split_count(nrb * (K / kSplitBN), kSplitGrid, N / kPK);
}

// Sum over splits s = 0, 1, ..., S - 1 (in that order) of outputs
// col .. col + 3 of listed row r (col a multiple of 4).  Split s holds all
// output tiles (column block major, then row block) at s * tiles tiles.
// The loads go out in groups of IN_FLIGHT, each group issued before its
// first add (16: one memory latency for any S, 64 registers of loads).
template <int IN_FLIGHT = 16>
__device__ __forceinline__ float4 split_sum4(const float *__restrict__ partial, int r, int col,
                                             int rows, int K, int S) {
    constexpr int kMaxSplit = 16;
    static_assert(kMaxSplit % IN_FLIGHT == 0, "groups of loads");
    const int nrb = (rows + kSplitBM - 1) / kSplitBM;
    const size_t stride = (size_t)nrb * (K / kSplitBN) * (kSplitBM * kSplitBN);
    const int tile = (col / kSplitBN) * nrb + r / kSplitBM;
    const float *src = partial + (size_t)tile * (kSplitBM * kSplitBN) + (r % kSplitBM) * kSplitBN +
                       col % kSplitBN;
    float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int g = 0; g < kMaxSplit; g += IN_FLIGHT) {
        if (g >= S) break;
        float4 v[IN_FLIGHT];
#pragma unroll
        for (int i = 0; i < IN_FLIGHT; ++i)
            if (g + i < S) v[i] = *reinterpret_cast<const float4 *>(src + (g + i) * stride);
#pragma unroll
        for (int i = 0; i < IN_FLIGHT; ++i)
            if (g + i < S) {
                if (g + i == 0) {
                    sum = v[0];
                } else {
                    sum.x += v[i].x;
                    sum.y += v[i].y;
                    sum.z += v[i].z;
                    sum.w += v[i].w;
                }
            }
    }
    return sum;
}

}  // namespace tw
