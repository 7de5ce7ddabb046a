// tw_gemm.hpp -- the software pipeline shared by the bf16 MFMA GEMMs:
// operands stream from global memory straight into LDS (buffer loads with
// the LDS bit, no register staging) through a ring of S stages, each 32
// reduction elements deep, several stages ahead of the multiplication.
#pragma once

#include "tw_device.hpp"

namespace tw {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kPK = 32;         // reduction depth of one pipeline stage
constexpr int kPRow = kPK * 2;  // 64 bytes per operand row in a stage

// Stage layout: operand row r occupies 64 bytes (4 chunks of 16 bytes);
// logical chunk kc lives at physical chunk kc ^ swz(r).  A fragment read
// (32 consecutive rows, one chunk per lane) then costs 4 LDS cycles per
// wave, the conflict-free minimum at 256 bytes per cycle; measured on gfx950
// with the SQ_LDS_BANK_CONFLICT counter, where XOR with ((r >> 1) ^ (r >> 3))
// or with (r & 7) on 128-byte rows still costs 8.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ uint32_t poff(int r, int kc) {
    return (uint32_t)(r * kPRow + ((kc ^ swz(r)) << 4));
}

// s_waitcnt lgkmcnt(0) with the other counters left alone.
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));
}

// s_waitcnt vmcnt(N) with the other counters left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `later` stages of NI direct loads each are still in
// flight (the loads of one wave complete in issue order).
template <int NI, int S>
__device__ __forceinline__ void wait_later(int later) {
    switch (later) {
    case 0: wait_vmcnt<0>(); break;
    case 1: if constexpr (S > 2) { wait_vmcnt<NI>(); break; } [[fallthrough]];
    case 2: if constexpr (S > 3) { wait_vmcnt<2 * NI>(); break; } [[fallthrough]];
    case 3: if constexpr (S > 4) { wait_vmcnt<3 * NI>(); break; } [[fallthrough]];
    case 4: if constexpr (S > 5) { wait_vmcnt<4 * NI>(); break; } [[fallthrough]];
    case 5: if constexpr (S > 6) { wait_vmcnt<5 * NI>(); break; } [[fallthrough]];
    default: if constexpr (S > 7) { wait_vmcnt<6 * NI>(); } else { wait_vmcnt<0>(); } break;
    }
}

// Scalar values the epilogue needs (kernel arguments) must be in registers
// before the k-loop.  Scalar loads and LDS reads share one completion
// counter and scalar loads may return out of order, so a scalar load still
// in flight inside the loop forces every LDS wait there to drain all reads
// (instead of only the older sub-step's), exposing the LDS latency before
// each batch of matrix instructions.  An empty asm that consumes the values
// makes their loads complete here.
template <typename P>
__device__ __forceinline__ void settle_scalar(P p) {
    asm volatile("" ::"s"(p));
}
template <typename... P>
__device__ __forceinline__ void settle_scalars(P... p) {
    (settle_scalar(p), ...);
}

// Output tile (bm, bn) of tile index t in an nbm x nbn grid, XCD-aware.
// Workgroups are dealt round-robin to the 8 XCDs (index % 8), and each XCD
// has its own L2.  When the grid splits evenly, XCD x gets one of RX x (8 /
// RX) regions of the grid, walked in groups of up to 8 row blocks column
// block by column block, so that the ~32 workgroups resident on one XCD
// share a few A row blocks and B column blocks in its L2.  Each A row block
// then comes into 8 / RX XCDs and each B column block into RX of them, so a
// GEMM whose A operand is the larger takes more row regions.  Otherwise the
// whole grid is walked in such groups.
template <int RX = 2>
__device__ __forceinline__ void xcd_tile(int t, int nbm, int nbn, int &bm, int &bn) {
    static_assert(RX == 1 || RX == 2 || RX == 4 || RX == 8, "regions of the 8 XCDs");
    constexpr int CX = 8 / RX;
    int r0m = 0, r0n = 0, rm = nbm, rn = nbn, local = t;
    if (nbm % RX == 0 && nbn % CX == 0) {
        const int x = t & 7;
        local = t >> 3;
        rm = nbm / RX;
        rn = nbn / CX;
        r0m = (x / CX) * rm;
        r0n = (x % CX) * rn;
    }
    constexpr int G = 8;
    const int group = local / (G * rn);
    const int gm = min(G, rm - group * G);
    const int ti = local - group * G * rn;
    bm = r0m + group * G + ti % gm;
    bn = r0n + ti / gm;
}

// The k-loop over stages [kt0, kt1) through a ring of S slots of
// `stage_bytes` at `ring`, with the LDS reads software-pipelined against the
// matrix instructions.  issue(kt, slot) enqueues this wave's NI direct loads
// of stage kt into `slot`.  Each stage has two sub-steps of 16 reduction
// elements; load(slot, sub, buf) reads one sub-step's fragments into
// register set buf (0 or 1) and mma(buf) issues its matrix instructions.
// The fragments of the next sub-step are always read before the current
// one's matrix instructions are issued, and the barrier of iteration i sits
// in the middle of stage i, after the first sub-step's matrix instructions.
// Before it every wave waits for its own loads of stage i + 1 (vector
// memory) and for its reads of stage i's second sub-step (LDS; they were
// issued a whole batch of matrix instructions earlier, so this wait is
// normally free).  The barrier therefore certifies that stage i + 1 is in
// LDS and that no wave reads stage i any more: after it the next stage's
// fragments may be read, and from iteration i + 1 on, stage i's slot may be
// refilled.
// A bare s_barrier is used: the fence of __syncthreads() would drain the
// loads still in flight.  The steady state (a stage still to issue) has no
// branches, so the compiler can wait for exactly the fragments each matrix
// instruction needs; a branch around the next stage's reads would make it
// wait for those too.  The last stages drain in a second loop.
template <int S, int NI, typename Issue, typename Load, typename Mma>
__device__ __forceinline__ void kloop_pipelined(int kt0, int kt1, char *ring, int stage_bytes,
                                                Issue issue, Load load, Mma mma) {
    static_assert(S >= 3 && S <= 8 && NI * (S - 2) < 64, "ring depth");
    const int n = kt1 - kt0;
    for (int j = 0; j < S - 1 && j < n; ++j) issue(kt0 + j, ring + (j % S) * stage_bytes);
    if (n <= 0) return;
    wait_later<NI, S>(min(S - 2, n - 1));  // stage 0 landed
    __builtin_amdgcn_s_barrier();
    load(ring, 0, 0);
    int i = 0;
    // sched_barrier(0) keeps the instruction scheduler from moving the
    // fragment reads behind the matrix instructions (which would fold the
    // two register sets into one and serialise reads and multiplies)
    for (; i + S - 1 < n; ++i) {
        load(ring + (i % S) * stage_bytes, 1, 1);
        issue(kt0 + i + S - 1, ring + ((i + S - 1) % S) * stage_bytes);  // slot of stage i - 1
        __builtin_amdgcn_sched_barrier(0);
        mma(0);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(S - 2) * NI>();  // stage i + 1 landed
        wait_lgkm0();                // stage i fully read
        __builtin_amdgcn_s_barrier();
        load(ring + ((i + 1) % S) * stage_bytes, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        mma(1);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (; i < n; ++i) {
        load(ring + (i % S) * stage_bytes, 1, 1);
        mma(0);
        if (i + 1 < n) {
            wait_later<NI, S>(n - 2 - i);
            wait_lgkm0();
            __builtin_amdgcn_s_barrier();
            load(ring + ((i + 1) % S) * stage_bytes, 0, 0);
        }
        mma(1);
    }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over `bytes` bytes at `base` (capped at 4 GiB - 1;
// a lane whose offset falls outside reads zeros).  Word 3 selects data
// format 32, which untyped buffer accesses need to be nonzero on gfx9-family
// parts.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint64_t bytes) {
    const uint32_t n = bytes < 0xffffffffull ? (uint32_t)bytes : 0xffffffffu;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}

// One wavefront-wide direct load: lane l copies the 16 bytes at byte
// voff + soff of the buffer to LDS dst + 16 l (dst wave-uniform, soff
// scalar).  The buffer form is used rather than the global one: the
// compiler books a global load-to-LDS as an access to both memories, and
// while one is in flight it turns every LDS wait into a wait for all
// outstanding LDS reads, so the fragments of the next sub-step could not be
// in flight across the current sub-step's matrix instructions.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, char *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, voff, soff, 0, 0);
}

// Lane offset for a 16-row x 64-byte stage load (1 KB): lane l writes
// physical chunk l % 4 of stage row row0 + l / 4, so it fetches the logical
// chunk that the swizzle puts there.  `row_off` is the byte offset of the
// lane's operand row in the buffer; the stage's reduction offset goes into
// the scalar offset of dma16.
__device__ __forceinline__ uint32_t rows16_voff(uint32_t row_off, int lane, int row0) {
    const int r = row0 + (lane >> 2);
    return row_off + (uint32_t)(((lane & 3) ^ swz(r)) << 4);
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i % 4
// of the 8-byte rows addressed by lanes 4 e + i / 4 (e = 0..3), a 4 x 4
// transpose of 16-bit elements.  The stages of the ring are ordered by
// explicit vector-memory waits and barriers.  Reads that carry no alias
// information are additionally made to wait for every direct load in flight
// (all later stages too); inlining this wrapper through a restrict-qualified
// pointer gives the read alias information like ordinary LDS loads have.
__device__ __forceinline__ i16x4 lds_tr16(const lds_i16x4 *__restrict__ p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_i16x4 *>(p));
}

// Fragment of v_mfma_f32_32x32x16_bf16 for sub-step s (0 or 1) of a stage:
// lane l reads row base + l % 32, reduction elements 16 s + 8 (l / 32) ...+7.
__device__ __forceinline__ u32x4 frag(const char *stage, int base, int s, int lane) {
    return lds_ld16(stage, poff(base + (lane & 31), 2 * s + (lane >> 5)));
}

}  // namespace tw
