// tw_device.hpp -- device helpers for the gfx950 kernels of the TwELL
// sparse gated-FFN forward: bf16 <-> fp32, the LDS tile layout used by every
// MFMA GEMM here, the bf16 MFMA wrapper and a DPP wavefront reduction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// One LDS stage holds BK = 64 reduction elements per tile row: 8 chunks of
// 16 bytes (8 bf16).  Chunk kc of row r lives at r*128 + ((kc ^ (r & 7)) * 16):
// the XOR swizzle puts the same logical chunk of 8 consecutive rows in 8
// different 16-byte bank groups, so the MFMA fragment reads (32 lanes, 32
// consecutive rows, one chunk each) and the 16-byte tile stores are free of
// bank conflicts.
constexpr int kBK = 64;
constexpr int kRowBytes = kBK * 2;

__device__ __forceinline__ uint32_t lds_off(int r, int kc) {
    return (uint32_t)(r * kRowBytes + ((kc ^ (r & 7)) << 4));
}

// --- bf16 helpers ----------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// --- global / LDS vector access --------------------------------------------
__device__ __forceinline__ u32x4 ld16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ void st16(void *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}
__device__ __forceinline__ u32x4 lds_ld16(const char *base, uint32_t off) {
    return *reinterpret_cast<const u32x4 *>(base + off);
}
__device__ __forceinline__ void lds_st16(char *base, uint32_t off, u32x4 v) {
    *reinterpret_cast<u32x4 *>(base + off) = v;
}

// --- MFMA ------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] * B[16x32].
// Operand lane layout: lane l holds row (l % 32) of A (resp. column (l % 32)
// of B) at reduction indices 8*(l/32) .. 8*(l/32)+7.
// Result lane layout: lane l, register i holds D[row][col] with
//   col = l % 32,  row = 8*(i/4) + 4*(l/32) + (i%4).
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ int mfma32_row(int i, int lane) {
    return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// --- wavefront sum (DPP) ----------------------------------------------------
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp0(float v) {
    // lanes with no source (outside the row, or rows masked off) read 0
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWMASK, 0xf, false));
}

// Sum of v over the 64 lanes, returned to every lane (fixed order, so the
// result is deterministic).  Inclusive scans within each 16-lane row
// (row_shr 1, 2, 4, 8), then row_bcast:15 and row_bcast:31 fold the rows into
// lane 63, which is broadcast.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp0<0x111, 0xf>(v);
    v += dpp0<0x112, 0xf>(v);
    v += dpp0<0x114, 0xf>(v);
    v += dpp0<0x118, 0xf>(v);
    v += dpp0<0x142, 0xa>(v);
    v += dpp0<0x143, 0xc>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Raise a kernel's dynamic LDS limit once per process: the first call sets
// the attribute and every later call returns that result (a function-local
// static is initialised exactly once, also when several host threads launch
// concurrently).
template <auto Kernel>
inline hipError_t lds_limit_once(int bytes) {
    static const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(Kernel), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    return e;
}

}  // namespace tw
