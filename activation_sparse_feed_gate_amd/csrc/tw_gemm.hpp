// tw_gemm.hpp -- the software pipeline shared by the bf16 MFMA GEMMs:
// operands stream from global memory straight into LDS (global_load_lds,
// no register staging) through a ring of 4 stages, each 32 reduction
// elements deep, so three stages are in flight while one is multiplied.
#pragma once

#include "tw_device.hpp"

namespace tw {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPK = 32;         // reduction depth of one pipeline stage
constexpr int kPRow = kPK * 2;  // 64 bytes per operand row in a stage
constexpr int kPStages = 4;

// Stage layout: operand row r occupies 64 bytes (4 chunks of 16 bytes);
// logical chunk kc lives at physical chunk kc ^ swz(r).  Across the 16 rows
// a fragment read touches in one LDS cycle the swizzle spreads the same
// logical chunk over all four chunk positions of both 128-byte halves.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
__device__ __forceinline__ uint32_t poff(int r, int kc) {
    return (uint32_t)(r * kPRow + ((kc ^ swz(r)) << 4));
}

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One wavefront-wide direct load: 16 operand rows x 64 bytes (1 KB) into LDS
// at `dst` (wave-uniform).  Lane l writes physical chunk l % 4 of row l / 4,
// so it fetches the logical chunk that the swizzle puts there.
// `src_row` points at the lane's operand row, `k` is the stage's first
// reduction element.
__device__ __forceinline__ void dma_rows16(const uint16_t *src_row, int k, int lane, int row0,
                                           char *dst) {
    const int r = row0 + (lane >> 2);
    const int kc = (lane & 3) ^ swz(r);
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src_row + k + kc * 8),
                                     (lds_void *)(dst), 16, 0, 0);
}

// Fragment of v_mfma_f32_32x32x16_bf16 for sub-step s (0 or 1) of a stage:
// lane l reads row base + l % 32, reduction elements 16 s + 8 (l / 32) ...+7.
__device__ __forceinline__ u32x4 frag(const char *stage, int base, int s, int lane) {
    return lds_ld16(stage, poff(base + (lane & 31), 2 * s + (lane >> 5)));
}

}  // namespace tw
