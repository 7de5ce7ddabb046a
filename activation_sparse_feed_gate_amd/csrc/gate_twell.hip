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
// - Macro tile 256 rows x 256 columns, 8 waves (two per SIMD, so one wave's
//   loads and LDS reads overlap the other's matrix work) in a 4 x 2 grid,
//   each wave owning 64 x 128 outputs as 2 x 4 blocks of
//   v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane).  Operands
//   stream from global memory straight into LDS (buffer loads with the LDS
//   bit, no register staging) through a 4-stage ring, 32 reduction elements
//   per stage, with the fragment reads software-pipelined against the matrix
//   instructions (tw_gemm.hpp).  Each XCD is given a compact region of the
//   tile grid so that its L2 serves the workgroups resident on it.
// - Epilogue: the ring is free after the k-loop.  Each wave stages 32 of its
//   64 rows of accumulators in LDS at a time; lane l then owns half a row
//   (row l % 32, 64 of the wave's 128 columns), builds its activity mask
//   (z > 0) with vector compares, and the two halves' popcounts give the
//   row count and this half's first slot, so the lane stores its entries in
//   ascending column order straight into TwELL.  No dense gate is written.
//   With T = 128 a tile is exactly one wave's 128 columns; with T = 256 it
//   spans the two waves of a wave row, which exchange their half counts
//   through LDS.  The 64 row counts of a wave are gathered into one register
//   (lane r holds row r) and stored by one instruction.
// - Each workgroup writes one bit per row (overflowing or not) for its column
//   block, so no buffer needs clearing beforehand; the compaction kernel ORs
//   the column blocks and lists the set rows in ascending order.
#include "tw_device.hpp"
#include "tw_gemm.hpp"
#include "tw_internal.hpp"

namespace tw {
namespace {

constexpr int kThreads = 512;                               // 8 waves, 2 per SIMD
constexpr int kStages = 4;
constexpr int kStageBytes = 2 * kGateBM * kPRow;            // A and B rows of one stage: 32 KB
constexpr int kRing = kStages * kStageBytes;                 // 128 KB ring
// Epilogue staging over the ring: per wave 32 rows x 128 fp32 columns, rows
// padded to 132 floats: 16 lanes reading the same columns of 16 different
// rows then touch 16 different 16-byte bank groups.
constexpr int kEpiPitch = 132;
constexpr int kEpiWave = 32 * kEpiPitch * 4;                 // 17 KB
constexpr int kLdsTiles = kRing > 8 * kEpiWave ? kRing : 8 * kEpiWave;
constexpr int kLdsBytes = kLdsTiles + 64 + 2 * kGateBM * 4; // + row flags + half counts

// PACK: the fused gate of the review (ReLU + TwELL packing in the epilogue,
// zdbg an optional debug copy of the gate).  !PACK: the unfused baseline's
// first half, the dense gate z written to zdbg and nothing packed (T unused).
template <int T, bool PACK>
__global__ __launch_bounds__(kThreads) void gate_twell_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg_t, int M, int K, int N,
    int C, int NBM, int NBN, float *__restrict__ tw_val, int32_t *__restrict__ tw_idx,
    int32_t *__restrict__ tw_cnt, uint32_t *__restrict__ oflag, float *__restrict__ zdbg) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint32_t *s_flag = reinterpret_cast<uint32_t *>(smem + kLdsTiles);
    int *s_half = reinterpret_cast<int *>(smem + kLdsTiles + 64);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;  // 4 x 2 waves, 64 x 128 outputs each
    int bm, bn;
    xcd_tile(blockIdx.x, NBM, NBN, bm, bn);
    const int m0 = bm * kGateBM, n0 = bn * kGateBN;

    if (tid < 8) s_flag[tid] = 0u;

    // Each wave streams rows [32 wave, 32 wave + 32) of both operands: two
    // 16-row direct loads per operand and stage (rows past M or N repeat the
    // last row; their results are never stored).
    const rsrc_t ra = make_rsrc(x + (size_t)m0 * K, (uint64_t)(M - m0) * K * 2);
    const rsrc_t rb = make_rsrc(wg_t + (size_t)n0 * K, (uint64_t)(N - n0) * K * 2);
    uint32_t aoff[2], boff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row0 = wave * 32 + j * 16;
        const int r = row0 + (lane >> 2);
        aoff[j] = rows16_voff((uint32_t)(min(m0 + r, M - 1) - m0) * K * 2, lane, row0);
        boff[j] = rows16_voff((uint32_t)(min(n0 + r, N - 1) - n0) * K * 2, lane, row0);
    }
    auto issue = [&](int kt, char *st) {
        const uint32_t soff = kt * kPK * 2;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row0 = wave * 32 + j * 16;
            dma16(ra, aoff[j], soff, st + row0 * kPRow);
            dma16(rb, boff[j], soff, st + (kGateBM + row0) * kPRow);
        }
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};

    u32x4 fa[2][2], fb[2][4];  // [register set][block]
    auto load = [&](const char *st, int s, int buf) {
        const char *bt = st + kGateBM * kPRow;
#pragma unroll
        for (int a = 0; a < 2; ++a) fa[buf][a] = frag(st, wm * 64 + a * 32, s, lane);
#pragma unroll
        for (int b = 0; b < 4; ++b) fb[buf][b] = frag(bt, wn * 128 + b * 32, s, lane);
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = mfma32(fa[buf][a], fb[buf][b], acc[a][b]);
    };
    settle_scalars(tw_val, tw_idx, tw_cnt, oflag, zdbg);
    kloop_pipelined<kStages, 4>(0, K / kPK, smem, kStageBytes, issue, load, mma);
    if constexpr (!PACK) {
        // each store instruction writes 32 consecutive columns of two rows
        const int ncol0 = n0 + wn * 128;
        if (ncol0 < N) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int m = m0 + wm * 64 + a * 32 + mfma32_row(i, lane);
                        if (m < M) zdbg[(size_t)m * N + ncol0 + b * 32 + (lane & 31)] = acc[a][b][i];
                    }
        }
        return;
    }
    __syncthreads();

    // ---------------- epilogue: ReLU + TwELL pack + row overflow bits ----
    // The ring is free after the main loop (the barrier above).  Each wave
    // stages 32 of its 64 rows at a time in LDS.  Lane l then owns half a
    // row: row l % 32, columns 64 (l / 32) ... +63 of this wave's 128.  It
    // builds the half-row's activity mask (z > 0) with vector compares, the
    // two halves' popcounts give the row count and this half's offset, and
    // the lane stores its entries in ascending column order.
    const int ncol0 = n0 + wn * 128;  // first column of this wave
    const bool live = ncol0 < N;      // false only in a half-empty last column block
    const int NT = N / T;
    const int t = ncol0 / T;
    const int wrow0 = m0 + wm * 64;   // first of the 64 rows this wave holds
    const int l32 = lane & 31, hc = lane >> 5;
    float *st = reinterpret_cast<float *>(smem + wave * kEpiWave);
    const float *rowp = st + l32 * kEpiPitch + hc * 64;

    int cnt_lane = 0;   // lane r: count of wave row r (this wave's columns or the whole tile)
    uint64_t over = 0;  // bit r: wave row r overflows (wave-uniform)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                st[mfma32_row(i, lane) * kEpiPitch + b * 32 + l32] = acc[a][b][i];
        if (zdbg && live) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = wrow0 + a * 32 + mfma32_row(i, lane);
                    if (m < M) zdbg[(size_t)m * N + ncol0 + b * 32 + l32] = acc[a][b][i];
                }
        }
        uint32_t mk[2] = {0u, 0u};
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const float4 v = *reinterpret_cast<const float4 *>(rowp + 4 * q);
            const uint32_t bits = (v.x > 0.0f ? 1u : 0u) | (v.y > 0.0f ? 2u : 0u) |
                                  (v.z > 0.0f ? 4u : 0u) | (v.w > 0.0f ? 8u : 0u);
            mk[q >> 3] |= bits << (4 * (q & 7));
        }
        const int cnt = __popc(mk[0]) + __popc(mk[1]);
        const int pcnt = __shfl_xor(cnt, 32);           // the other half of the row
        int total = cnt + pcnt;                          // this wave's 128 columns
        int off = hc ? pcnt : 0;                         // entries before this half
        const int rw = a * 32 + l32;                     // wave row of this lane
        const int m = wrow0 + rw;
        if (T == 256) {
            // the two waves of a wave row hold the two halves of each tile
            if (hc == 0) s_half[wn * kGateBM + wm * 64 + rw] = total;
            __syncthreads();
            const int other = s_half[(wn ^ 1) * kGateBM + wm * 64 + rw];
            if (wn) off += other;
            total += other;
        }
        if (live && m < M && off < C) {
            const size_t tb = ((size_t)m * NT + t) * C;
            uint64_t bits = (uint64_t)mk[0] | ((uint64_t)mk[1] << 32);
            int slot = off;
            while (bits && slot < C) {
                const int c = __builtin_ctzll(bits);
                bits &= bits - 1;
                tw_idx[tb + slot] = ncol0 + hc * 64 + c;
                tw_val[tb + slot] = rowp[c];
                ++slot;
            }
        }
        // every lane joins the shuffle: a permute reading an inactive lane
        // yields 0, so it must not sit under the select below
        const int tsh = __shfl(total, lane & 31);
        cnt_lane = (lane >> 5) == a ? tsh : cnt_lane;
        // rows past M repeat row M-1 and must not be routed
        const uint64_t ov = __ballot(hc == 0 && total > C && m < M);
        over |= (ov & 0xffffffffull) << (32 * a);
        if (T == 256) __syncthreads();  // s_half is rewritten for the next 32 rows
    }
    const bool owner = T == 128 || wn == 0;  // the wave that stores this tile's counts
    if (owner && live) {
        if (wrow0 + lane < M) tw_cnt[(size_t)(wrow0 + lane) * NT + t] = cnt_lane;
        if (lane == 0 && over) {
            if ((uint32_t)over) atomicOr(&s_flag[wm * 2], (uint32_t)over);
            if ((uint32_t)(over >> 32)) atomicOr(&s_flag[wm * 2 + 1], (uint32_t)(over >> 32));
        }
    }
    __syncthreads();
    const int MW = (M + 31) >> 5;
    if (tid < 8 && m0 + 32 * tid < M) oflag[(size_t)bn * MW + (m0 >> 5) + tid] = s_flag[tid];
}

// ------------------------- small batches (decode) ---------------------------
// With few token rows the 256-row macro tile is mostly padding, so its
// matrix work, not the weights, sets the time (and only N / 256 workgroups
// run).  This variant takes 64 rows x one TwELL tile (T columns) per
// workgroup of 4 waves: every wave holds the 64 rows x T / 4 columns, the
// operands stream through the same 4-stage direct-to-LDS ring, and the
// epilogue stages the 64 x T tile in LDS and packs one row at a time per
// wave (lane l holds T / 64 consecutive columns; a wave-wide scan of the
// lanes' counts gives the slots in ascending column order).  The row
// overflow bits go to oflag[tile][row word]: N / T column blocks.
// Such workgroups number NRB N / T (NRB 64-row blocks); each streams its
// slice of W_g through one CU.  By how many there are (counted at T = 128
// for every T, so that the fused gate and the unfused dense gate take the
// same route and sum z in the same order):
// - under 128, and few rows (the partial gates small next to W_g): the
//   reduction is split over S workgroups (S = 2, 4 or 8 K-slices) that write
//   fp32 partial tiles to the workspace, and a second kernel sums them in
//   slice order and packs (the whole chip streams W_g);
// - under 256: each workgroup holds KS = 2 groups of 4 waves that take the
//   two halves of the reduction through their own rings and add in LDS;
// - else one group, the whole reduction.
constexpr int kSmallBM = 64;

// Workgroups of the small-batch gate, counted at T = 128.
inline long long gate_small_wg(int M, int N) {
    return (long long)((M + kSmallBM - 1) / kSmallBM) * (N / 128);
}
// K-slices of the split reduction (1: none): enough for 256 to 512
// workgroups, at most 8, dividing the K / 32 stages; taken only while the
// partial gates (S M N fp32, written and read back) stay within an eighth of
// W_g's bytes (S M 16 <= K).  Measured: at M = 1 and 16 of the 2B block the
// gate took 10.8 and 16.5 us split against 21.5 and 23.9 whole; past that
// bound (M = 16 and 64 at the 0.5B block, 64 at the 2B) the partials cost more.
inline int gate_small_parts(int M, int N, int K) {
    if (!gate_small(M, N)) return 1;
    const long long wg = gate_small_wg(M, N);
    if (wg >= 128) return 1;
    int S = 8;
    while (S > 2 && (wg * S > 256 * 2 || (K / kPK) % S)) S >>= 1;
    if ((K / kPK) % S || (long long)S * M * 16 > K) return 1;
    return S;
}
// Whether the workgroups of the unsplit small-batch gate take two K halves.
inline bool gate_small_split(int M, int N, int K) {
    return gate_small_parts(M, N, K) == 1 && gate_small_wg(M, N) < 256;
}

template <int T, int KS>
struct SmallGate {
    static constexpr int NW = 4, WC = T / NW;          // waves per group, columns per wave
    static constexpr int NTH = KS * NW * 64;            // threads
    static constexpr int FB = WC / 32;                  // 32-column blocks per wave
    static constexpr int SR = kSmallBM + T;             // stage rows: x, then W_g
    static constexpr int NI = SR / (16 * NW);           // direct loads per wave and stage
    static constexpr int STAGE = SR * kPRow;
    static constexpr int ST = kStages;                  // ring stages per group
    static constexpr int RING = ST * STAGE;             // one group's ring
    static constexpr int PITCH = T + 4;                 // staged row, floats
    static constexpr int EPI = kSmallBM * PITCH * 4;    // staged tile, then 2 flag words
    static constexpr int LDS = KS * RING > EPI + 16 ? KS * RING : EPI + 16;
    static_assert(SR % (16 * NW) == 0 && kSmallBM % (16 * NW) == 0, "load slots");
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(NTH == 256 * KS, "launch bounds of gate_small_kernel");
};

// Pack the staged 64 x T tile zs (rows of PITCH floats) of row block m0 and
// tile tc: TwELL slots, counts and row overflow bits (and the dense copy
// zdbg when given; tw_cnt null: only that copy).  NWAVES waves share the
// rows; s_flag (2 words, zero) collects the block's overflow bits.  Ends
// with the block's oflag words written.
template <int T, int NWAVES>
__device__ __forceinline__ void pack_tile(const float *zs, int pitch, uint32_t *s_flag,
                                          int wave, int lane, int tid, int m0, int n0, int tc,
                                          int M, int N, int C, float *__restrict__ tw_val,
                                          int32_t *__restrict__ tw_idx,
                                          int32_t *__restrict__ tw_cnt,
                                          uint32_t *__restrict__ oflag,
                                          float *__restrict__ zdbg) {
    constexpr int CPL = T / 64;  // columns per lane
    const int NT = N / T;
    uint64_t over = 0;           // bit r: row r of the block overflows (wave-uniform)
    for (int r = wave; r < kSmallBM; r += NWAVES) {
        const int m = m0 + r;
        if (m >= M) break;  // wave-uniform
        float v[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) v[k] = zs[r * pitch + lane * CPL + k];
        if (zdbg) {
#pragma unroll
            for (int k = 0; k < CPL; ++k) zdbg[(size_t)m * N + n0 + lane * CPL + k] = v[k];
        }
        if (!tw_cnt) continue;  // the dense gate only (the unfused path's first half)
        uint32_t bits = 0;
#pragma unroll
        for (int k = 0; k < CPL; ++k) bits |= (v[k] > 0.0f ? 1u : 0u) << k;
        const int cnt = __popc(bits);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(incl, d);
            if (lane >= d) incl += u;
        }
        const int total = __shfl(incl, 63);
        const size_t tb = ((size_t)m * NT + tc) * C;
        int slot = incl - cnt;
#pragma unroll
        for (int k = 0; k < CPL; ++k)
            if ((bits >> k) & 1u) {
                if (slot < C) {
                    tw_idx[tb + slot] = n0 + lane * CPL + k;
                    tw_val[tb + slot] = v[k];
                }
                ++slot;
            }
        if (lane == 0) tw_cnt[(size_t)m * NT + tc] = total;
        if (total > C) over |= 1ull << r;
    }
    if (lane == 0 && over) {
        if ((uint32_t)over) atomicOr(&s_flag[0], (uint32_t)over);
        if ((uint32_t)(over >> 32)) atomicOr(&s_flag[1], (uint32_t)(over >> 32));
    }
    __syncthreads();
    const int MW = (M + 31) >> 5;
    if (oflag && tid < 2 && m0 + 32 * tid < M)
        oflag[(size_t)tc * MW + (m0 >> 5) + tid] = s_flag[tid];
}

// PART = false: the fused gate (or, with tw_cnt null, the dense gate into
// zdbg).  The reduction runs as `nseq` consecutive K-slices, each from zero,
// added in slice order (the order the split path sums its partial tiles in;
// nseq = 1 otherwise), by KS groups of waves (two halves when KS = 2).
// PART = true: workgroup (tile, slice) reduces K-slice `slice` of `nseq` and
// stores the fp32 partial tile to part[slice][M][N].
template <int T, int KS, bool PART>
__global__ __launch_bounds__(256 * KS) void gate_small_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg_t, int M, int K, int N,
    int C, int NRB, int nseq, float *__restrict__ tw_val, int32_t *__restrict__ tw_idx,
    int32_t *__restrict__ tw_cnt, uint32_t *__restrict__ oflag, float *__restrict__ zdbg,
    float *__restrict__ part) {
    using P = SmallGate<T, KS>;
    static_assert(!PART || KS == 1, "one group per K-slice");
    extern __shared__ __attribute__((aligned(16))) char smem[];
    uint32_t *s_flag = reinterpret_cast<uint32_t *>(smem + P::EPI);  // after the k-loop only
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave_all / P::NW, wave = wave_all % P::NW;  // K half, wave in the group
    const int NT = N / T;
    const int tile = PART ? blockIdx.x % (NRB * NT) : blockIdx.x;
    const int slice = PART ? blockIdx.x / (NRB * NT) : 0;
    const int rb = tile % NRB, tc = tile / NRB;  // row block, tile
    const int m0 = rb * kSmallBM, n0 = tc * T;

    // load slot j of a wave: stage rows [16 (4 j + wave), +16); slot 0 is x
    const rsrc_t ra = make_rsrc(x + (size_t)m0 * K, (uint64_t)(M - m0) * K * 2);
    const rsrc_t rw = make_rsrc(wg_t + (size_t)n0 * K, (uint64_t)T * K * 2);
    uint32_t voff[P::NI];
#pragma unroll
    for (int j = 0; j < P::NI; ++j) {
        const int row0 = (j * P::NW + wave) * 16;
        const int sr = row0 + (lane >> 2);
        const uint32_t row_off = j == 0 ? (uint32_t)(min(m0 + sr, M - 1) - m0) * K * 2
                                        : (uint32_t)(sr - kSmallBM) * K * 2;
        voff[j] = rows16_voff(row_off, lane, row0);
    }
    auto issue = [&](int kt, char *st) {
        const uint32_t soff = kt * kPK * 2;
#pragma unroll
        for (int j = 0; j < P::NI; ++j) {
            const int row0 = (j * P::NW + wave) * 16;
            if (j == 0) dma16(ra, voff[j], soff, st + row0 * kPRow);
            else dma16(rw, voff[j], soff, st + row0 * kPRow);
        }
    };
    f32x16 acc[2][P::FB], tot[2][P::FB];
    u32x4 fa[2][2], fb[2][P::FB];
    auto load = [&](const char *st, int s, int buf) {
#pragma unroll
        for (int a = 0; a < 2; ++a) fa[buf][a] = frag(st, a * 32, s, lane);
#pragma unroll
        for (int b = 0; b < P::FB; ++b)
            fb[buf][b] = frag(st, kSmallBM + wave * P::WC + b * 32, s, lane);
    };
    auto mma = [&](int buf) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b) acc[a][b] = mfma32(fa[buf][a], fb[buf][b], acc[a][b]);
    };
    settle_scalars(tw_val, tw_idx, tw_cnt, oflag, zdbg, part);
    // K-slices of kts stages; with KS = 2, group g takes half g of each
    // (both groups run the same number of stages, so the ring's
    // workgroup-wide barriers pair up)
    const int kts = K / kPK / nseq, kth = kts / KS;
    const int q0 = PART ? slice : 0, q1 = PART ? slice + 1 : nseq;
    for (int q = q0; q < q1; ++q) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b) acc[a][b] = f32x16{};
        const int k0 = q * kts + grp * kth;
        kloop_pipelined<P::ST, P::NI>(k0, k0 + kth, smem + grp * P::RING, P::STAGE, issue, load,
                                      mma);
        __syncthreads();  // the ring is free again
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b) {
                if (q == q0) tot[a][b] = acc[a][b];
                else
#pragma unroll
                    for (int i = 0; i < 16; ++i) tot[a][b][i] += acc[a][b][i];
            }
    }
    if constexpr (PART) {
        // the partial tile, one 32-column block per store instruction
        float *pt = part + (size_t)slice * M * N;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int m = m0 + a * 32 + mfma32_row(i, lane);
                    if (m < M) pt[(size_t)m * N + n0 + wave * P::WC + b * 32 + (lane & 31)] = tot[a][b][i];
                }
        return;
    }

    float *zs = reinterpret_cast<float *>(smem);
    auto zo = [&](int a, int b, int i) {
        return (a * 32 + mfma32_row(i, lane)) * P::PITCH + wave * P::WC + b * 32 + (lane & 31);
    };
    if (grp == 0) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i) zs[zo(a, b, i)] = tot[a][b][i];
    }
    if (tid < 2) s_flag[tid] = 0u;
    __syncthreads();
    if constexpr (KS == 2) {
        // z = (first half) + (second half), added by the lane that holds
        // the same element in the second group
        if (grp == 1) {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < P::FB; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) zs[zo(a, b, i)] += tot[a][b][i];
        }
        __syncthreads();
    }
    pack_tile<T, KS * P::NW>(zs, P::PITCH, s_flag, wave_all, lane, tid, m0, n0, tc, M, N, C,
                             tw_val, tw_idx, tw_cnt, oflag, zdbg);
}

// The split path's second pass: workgroup (row block, tile) sums the S
// partial tiles in slice order into the LDS staging and packs the tile.
template <int T>
__global__ __launch_bounds__(256) void gate_sumpack_kernel(
    const float *__restrict__ part, int S, int M, int N, int C, int NRB,
    float *__restrict__ tw_val, int32_t *__restrict__ tw_idx, int32_t *__restrict__ tw_cnt,
    uint32_t *__restrict__ oflag, float *__restrict__ zdbg) {
    using P = SmallGate<T, 1>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    float *zs = reinterpret_cast<float *>(smem);
    uint32_t *s_flag = reinterpret_cast<uint32_t *>(smem + P::EPI);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rb = blockIdx.x % NRB, tc = blockIdx.x / NRB;
    const int m0 = rb * kSmallBM, n0 = tc * T;
    const int rows = min(kSmallBM, M - m0);
    constexpr int C4 = T / 4;  // float4 per tile row
    constexpr int kMaxS = 8;   // gate_small_parts takes at most 8 slices
    for (int q = tid; q < rows * C4; q += 256) {
        const int r = q / C4, c = 4 * (q % C4);
        const float *src = part + (size_t)(m0 + r) * N + n0 + c;
        // every slice's load issued before the first add (one latency)
        float4 u[kMaxS];
#pragma unroll
        for (int s = 0; s < kMaxS; ++s)
            if (s < S) u[s] = *reinterpret_cast<const float4 *>(src + (size_t)s * M * N);
        float4 v = u[0];
#pragma unroll
        for (int s = 1; s < kMaxS; ++s)
            if (s < S) {
                v.x += u[s].x;
                v.y += u[s].y;
                v.z += u[s].z;
                v.w += u[s].w;
            }
        *reinterpret_cast<float4 *>(zs + r * P::PITCH + c) = v;
    }
    if (tid < 2) s_flag[tid] = 0u;
    __syncthreads();
    pack_tile<T, 4>(zs, P::PITCH, s_flag, wave, lane, tid, m0, n0, tc, M, N, C, tw_val, tw_idx,
                    tw_cnt, oflag, zdbg);
}

template <int T, int KS, bool PART>
hipError_t launch_small(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N, int C,
                        int nseq, float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                        uint32_t *oflag, float *z_debug, float *part, hipStream_t s) {
    using P = SmallGate<T, KS>;
    {
        const hipError_t e = lds_limit_once<&gate_small_kernel<T, KS, PART>>(P::LDS);
        if (e != hipSuccess) return e;
    }
    const int NRB = (M + kSmallBM - 1) / kSmallBM;
    const int grid = NRB * (N / T) * (PART ? nseq : 1);
    hipLaunchKernelGGL((gate_small_kernel<T, KS, PART>), dim3(grid), dim3(P::NTH), P::LDS, s, x,
                       wg_t, M, K, N, C, NRB, nseq, tw_val, tw_idx, tw_cnt, oflag, z_debug, part);
    return hipGetLastError();
}

// The fused small-batch gate: split path (partials, then sum + pack), two K
// halves per workgroup, or one.  `part`: gate_part_bytes(M, K, N) bytes.
template <int T>
hipError_t launch_gate_small(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N, int C,
                             float *tw_val, int32_t *tw_idx, int32_t *tw_cnt, uint32_t *oflag,
                             float *z_debug, float *part, hipStream_t s) {
    const int S = gate_small_parts(M, N, K);
    if (S > 1) {
        hipError_t e = launch_small<T, 1, true>(x, wg_t, M, K, N, C, S, nullptr, nullptr, nullptr,
                                                nullptr, nullptr, part, s);
        if (e != hipSuccess) return e;
        using P = SmallGate<T, 1>;
        e = lds_limit_once<&gate_sumpack_kernel<T>>(P::EPI + 16);
        if (e != hipSuccess) return e;
        const int NRB = (M + kSmallBM - 1) / kSmallBM;
        hipLaunchKernelGGL(gate_sumpack_kernel<T>, dim3(NRB * (N / T)), dim3(256), P::EPI + 16, s,
                           part, S, M, N, C, NRB, tw_val, tw_idx, tw_cnt, oflag, z_debug);
        return hipGetLastError();
    }
    if (gate_small_split(M, N, K))
        return launch_small<T, 2, false>(x, wg_t, M, K, N, C, 1, tw_val, tw_idx, tw_cnt, oflag,
                                         z_debug, nullptr, s);
    return launch_small<T, 1, false>(x, wg_t, M, K, N, C, 1, tw_val, tw_idx, tw_cnt, oflag,
                                     z_debug, nullptr, s);
}

// Ascending list of the rows whose bit is set in any column block.  One
// workgroup of 512 threads, 512 words (16384 rows) at a time: thread t ORs
// word base + t over the column blocks itself (consecutive threads read
// consecutive words of a block, and up to 32 blocks' loads are in flight
// before any is used, so a chunk costs one memory round trip up to 32
// column blocks), then a block-wide scan of the words' popcounts gives every
// set bit its list position.
constexpr int kCompactThreads = 512;
constexpr int kCompactLoads = 32;  // column blocks loaded together

__global__ __launch_bounds__(kCompactThreads) void ovf_compact_kernel(
    const uint32_t *__restrict__ oflag, int NB, int MW, int R_max,
    int32_t *__restrict__ ovf_rows, int32_t *__restrict__ ovf_count) {
    constexpr int kWaves = kCompactThreads / 64;
    __shared__ int s_wsum[kWaves];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    int running = 0;
    for (int base = 0; base < MW; base += kCompactThreads) {
        const int w = base + tid;
        uint32_t word = 0u;
        if (w < MW) {
            for (int b0 = 0; b0 < NB; b0 += kCompactLoads) {
                uint32_t v[kCompactLoads];
#pragma unroll
                for (int u = 0; u < kCompactLoads; ++u)
                    v[u] = b0 + u < NB ? oflag[(size_t)(b0 + u) * MW + w] : 0u;
#pragma unroll
                for (int u = 0; u < kCompactLoads; ++u) word |= v[u];
            }
        }
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
#pragma unroll
        for (int q = 0; q < kWaves; ++q) {
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
        __syncthreads();  // s_wsum is rewritten for the next chunk
    }
    if (tid == 0) *ovf_count = running;
}

template <int T, bool PACK>
hipError_t launch_gate_t(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N, int C,
                         float *tw_val, int32_t *tw_idx, int32_t *tw_cnt, uint32_t *oflag,
                         float *z_debug, hipStream_t s) {
    {
        const hipError_t e = lds_limit_once<&gate_twell_kernel<T, PACK>>(kLdsBytes);
        if (e != hipSuccess) return e;
    }
    const int NBN = gate_col_blocks(N);
    const int NBM = (M + kGateBM - 1) / kGateBM;
    hipLaunchKernelGGL((gate_twell_kernel<T, PACK>), dim3(NBN * NBM), dim3(kThreads), kLdsBytes,
                       s, x, wg_t, M, K, N, C, NBM, NBN, tw_val, tw_idx, tw_cnt, oflag, z_debug);
    return hipGetLastError();
}

}  // namespace

int gate_flag_blocks(int M, int N, int T) {
    return gate_small(M, N) ? N / T : gate_col_blocks(N);
}

size_t gate_part_bytes(int M, int K, int N) {
    const int S = gate_small_parts(M, N, K);
    return S > 1 ? (size_t)S * M * N * sizeof(float) : 0;
}

hipError_t launch_gate_twell(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N,
                             int T, int C, float *tw_val, int32_t *tw_idx, int32_t *tw_cnt,
                             uint32_t *oflag, float *z_debug, float *part, hipStream_t s) {
    if (M == 0) return hipSuccess;
    if (gate_small(M, N)) {
        if (T == 128)
            return launch_gate_small<128>(x, wg_t, M, K, N, C, tw_val, tw_idx, tw_cnt, oflag,
                                          z_debug, part, s);
        return launch_gate_small<256>(x, wg_t, M, K, N, C, tw_val, tw_idx, tw_cnt, oflag, z_debug,
                                      part, s);
    }
    if (T == 128)
        return launch_gate_t<128, true>(x, wg_t, M, K, N, C, tw_val, tw_idx, tw_cnt, oflag,
                                        z_debug, s);
    return launch_gate_t<256, true>(x, wg_t, M, K, N, C, tw_val, tw_idx, tw_cnt, oflag, z_debug,
                                    s);
}

hipError_t launch_gate_dense(const uint16_t *x, const uint16_t *wg_t, int M, int K, int N,
                             float *z, hipStream_t s) {
    if (M == 0) return hipSuccess;
    // the summation order tw_pack_gate would take, so that z is the same to
    // the bit: its K-slices (added in slice order, here within each
    // workgroup, so no workspace is needed) or its two K halves
    if (gate_small(M, N)) {
        const int S = gate_small_parts(M, N, K);
        if (S > 1)
            return launch_small<128, 1, false>(x, wg_t, M, K, N, 1, S, nullptr, nullptr, nullptr,
                                               nullptr, z, nullptr, s);
        if (gate_small_split(M, N, K))
            return launch_small<128, 2, false>(x, wg_t, M, K, N, 1, 1, nullptr, nullptr, nullptr,
                                               nullptr, z, nullptr, s);
        return launch_small<128, 1, false>(x, wg_t, M, K, N, 1, 1, nullptr, nullptr, nullptr,
                                           nullptr, z, nullptr, s);
    }
    return launch_gate_t<128, false>(x, wg_t, M, K, N, 1, nullptr, nullptr, nullptr, nullptr, z,
                                     s);
}

hipError_t launch_ovf_compact(const uint32_t *oflag, int NB, int MW, int R_max,
                              int32_t *ovf_rows, int32_t *ovf_count, hipStream_t s) {
    hipLaunchKernelGGL(ovf_compact_kernel, dim3(1), dim3(kCompactThreads), 0, s, oflag, NB, MW,
                       R_max, ovf_rows, ovf_count);
    return hipGetLastError();
}

}  // namespace tw
