// dense_ffn.hip -- dense gated FFN on bf16 MFMA: the dense backup of the
// rows that overflow a TwELL tile, and the all-rows dense comparator.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 1-1 equation (h_u = x W_u, h_g = ReLU(x W_g), h = h_u * h_g,
// y = h W_d) and section 3-6 (rows over capacity keep their full activation
// through a dense path on the matrix cores instead of being clipped).
//
// gfx950 design
// - Both GEMMs stream their operands from global memory straight into LDS
//   through the 4-stage ring of tw_gemm.hpp (32 reduction elements a stage).
// - gate+up: one GEMM with two B operands, so x is read once for both; the
//   epilogue forms h = ReLU(g) * u and rounds it to bf16 (g and u are never
//   stored).  Workgroups loop over tiles: the overflow path sizes its grid
//   for the capacity and finds the actual number of rows on the device.
// - down: A = h [rows][N] (reduction-contiguous), B = W_d [N][K], whose
//   reduction index is its row index.  W_d rows land in LDS in their natural
//   layout and the MFMA B fragments are read with ds_read_b64_tr_b16, the
//   gfx950 LDS read that transposes 16-bit elements across a 16-lane group.
// - With few rows (the overflow path) the down GEMM also splits the
//   reduction over N so that every CU has work; each split writes a partial
//   tile and the partials are summed in split order (the result does not
//   depend on timing) by a small kernel, or, for the inference path's
//   overflow rows, by the sparse kernel that runs next (tw_split.hpp).  A
//   device-scope fence per workgroup instead would write back the whole L2
//   of its XCD each time.
// - Rows come either directly or through a row list with a device-side
//   count (the overflow list): x rows are gathered and y rows scattered
//   through it.
#include "tw_device.hpp"
#include "tw_gemm.hpp"
#include "tw_internal.hpp"
#include "tw_split.hpp"

namespace tw {
namespace {

// Rows to process: the device-side count (capped) or R_cap.  Read into a
// scalar register: buffer descriptors built from it must be wave-uniform.
__device__ __forceinline__ int rows_of(const int32_t *count, int R_cap) {
    return __builtin_amdgcn_readfirstlane(count ? min(*count, R_cap) : R_cap);
}

// ------------------------------ gate + up ---------------------------------
template <int BM, int BN, int WM, int WN, int S, int NB = 2>
struct GU {
    static constexpr int NW = WM * WN, NTH = NW * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
    static constexpr int FA = TM / 32, FB = TN / 32;  // 32-blocks per wave
    static constexpr int SR = BM + NB * BN;           // stage rows: A, then W_g (, then W_u)
    static constexpr int NI = SR / (16 * NW);         // direct loads per wave and stage
    static constexpr int STAGE = SR * kPRow;
    static constexpr int LDS = S * STAGE;
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
    // each wave's 16-row load slice lies in one operand (the operand is then
    // wave-uniform), and the stage splits evenly over the waves
    static_assert(BM % 16 == 0 && BN % 16 == 0 && SR % (16 * NW) == 0, "load slices");
};

// Segment sg of the sparse kernel's heaviest-first row order (RowOrder):
// one row per thread, its counts read in one round of loads; a block-wide
// ordered compaction puts the segment's heavy rows first.
template <int NTH>
__device__ void row_order_block(const RowOrder &o, int sg, char *smem) {
    static_assert(NTH >= kOrderSeg, "one row per thread");
    constexpr int NW = NTH / 64;
    int *s_w = reinterpret_cast<int *>(smem);  // 2 NW wave counts
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = sg * kOrderSeg;
    const int nrows = min(kOrderSeg, o.M - r0);
    const bool in = tid < nrows;
    bool heavy = false;
    if (in) {
        const int32_t *cr = o.tw_cnt + (size_t)(r0 + tid) * o.NT;
        int tot = 0;
        bool over = false;
        if ((o.NT & 3) == 0) {
#pragma unroll 8
            for (int t = 0; t < o.NT; t += 4) {
                const int4 c = *reinterpret_cast<const int4 *>(cr + t);
                tot += c.x + c.y + c.z + c.w;
                over |= (c.x > o.C) | (c.y > o.C) | (c.z > o.C) | (c.w > o.C);
            }
        } else {
            for (int t = 0; t < o.NT; ++t) {
                tot += cr[t];
                over |= cr[t] > o.C;
            }
        }
        heavy = !over && tot > o.H;
    }
    const uint64_t bh = __ballot(heavy), bl = __ballot(in && !heavy);
    if (lane == 0) {
        s_w[wave] = __popcll(bh);
        s_w[NW + wave] = __popcll(bl);
    }
    __syncthreads();
    int hb = 0, lb = 0, ht = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int a = s_w[w], b = s_w[NW + w];
        hb += w < wave ? a : 0;
        lb += w < wave ? b : 0;
        ht += a;
    }
    const uint64_t below = (1ull << lane) - 1;
    int32_t *slots = o.perm + 128 + r0;
    if (heavy) slots[hb + __popcll(bh & below)] = r0 + tid;
    else if (in) slots[ht + lb + __popcll(bl & below)] = r0 + tid;
    if (tid == 0) {
        o.perm[sg] = ht;
        o.perm[64 + sg] = nrows - ht;
    }
}

// Epilogue modes:
//   kGU    h = bf16(ReLU(g) u)
//   kKeep  h, and bf16(ReLU(g)) / bf16(u) into g_out / u_out where given
//          (the dense backup rows of the hybrid training storage keep both)
//   kDh    one weight operand (wg_t = W_d, x = dy): dh = dy_r . W_d[n], then
//          with the stored bf16 gate and up values of the row (g_in, u_in):
//          h <- bf16(dh g) (du) and g_out <- bf16(g > 0 ? dh u + l1 : 0) (dz)
enum { kGU = 0, kKeep = 1, kDh = 2 };

template <int BM, int BN, int WM, int WN, int S, int MODE>
__global__ __launch_bounds__(WM * WN * 64) void gateup_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg_t,
    const uint16_t *__restrict__ wu_t, int K, int N, const int32_t *__restrict__ rowlist,
    const int32_t *__restrict__ count, int R_cap, int xrows, uint16_t *__restrict__ h,
    uint16_t *__restrict__ g_out, uint16_t *__restrict__ u_out,
    const uint16_t *__restrict__ g_in, const uint16_t *__restrict__ u_in, float l1,
    RowOrder ord) {
    constexpr int NB = MODE == kDh ? 1 : 2;  // weight operands
    using P = GU<BM, BN, WM, WN, S, NB>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    // the last workgroups write the sparse kernel's row order, when asked
    const int nseg = ord.perm ? row_order_segs(ord.M) : 0;
    const int gridw = gridDim.x - nseg;  // the GEMM's workgroups
    if ((int)blockIdx.x >= gridw) {
        row_order_block<P::NTH>(ord, blockIdx.x - gridw, smem);
        return;
    }

    const int rows = rows_of(count, R_cap);
    const int nrb = (rows + BM - 1) / BM;
    const int ntiles = nrb * (N / BN);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31;
    const int KT = K / kPK;

    const int ncb = N / BN;
    for (int t = blockIdx.x; t < ntiles; t += gridw) {
        int rb, cb;
        if (rowlist) {
            // few rows: all row blocks of a weight column block on one XCD
            // (workgroup index % 8), so the weights are fetched once per XCD
            if ((ncb & 7) == 0 && (gridw & 7) == 0) {
                const int local = t >> 3;
                cb = (local / nrb) * 8 + (t & 7);
                rb = local % nrb;
            } else {
                rb = t % nrb;
                cb = t / nrb;
            }
        } else {
            xcd_tile(t, nrb, ncb, rb, cb);
        }
        const int m0 = rb * BM, n0 = cb * BN;
        // x rows come through the row list (any of the xrows rows) or are
        // the tile's own; the weight rows are the column block's
        const uint16_t *xb = rowlist ? x : x + (size_t)m0 * K;
        const uint64_t xbytes = (uint64_t)(rowlist ? xrows : rows - m0) * K * 2;
        const uint16_t *gb = wg_t + (size_t)n0 * K;
        const uint16_t *ub = NB == 2 ? wu_t + (size_t)n0 * K : gb;
        // Load j of a wave fetches stage rows [16 (j NW + wave), +16), all in
        // one operand (BM and BN are multiples of 16), chosen per wave.
        uint32_t voff[P::NI];
#pragma unroll
        for (int j = 0; j < P::NI; ++j) {
            const int row0 = (j * P::NW + wave) * 16;
            const int sr = row0 + (lane >> 2);
            uint32_t row_off;
            if (row0 < BM) {
                const int r = min(m0 + sr, rows - 1);
                row_off = rowlist ? (uint32_t)rowlist[r] * K * 2 : (uint32_t)(r - m0) * K * 2;
            } else if (NB == 1 || row0 < BM + BN) {
                row_off = (uint32_t)(sr - BM) * K * 2;
            } else {
                row_off = (uint32_t)(sr - BM - BN) * K * 2;
            }
            voff[j] = rows16_voff(row_off, lane, row0);
        }
        const rsrc_t rx = make_rsrc(xb, xbytes);
        const rsrc_t rg = make_rsrc(gb, (uint64_t)BN * K * 2);
        const rsrc_t ru = make_rsrc(ub, (uint64_t)BN * K * 2);
        auto issue = [&](int kt, char *st) {
            const uint32_t soff = kt * kPK * 2;
#pragma unroll
            for (int j = 0; j < P::NI; ++j) {
                const int row0 = (j * P::NW + wave) * 16;
                char *dst = st + row0 * kPRow;
                if (row0 < BM) dma16(rx, voff[j], soff, dst);
                else if (NB == 1 || row0 < BM + BN) dma16(rg, voff[j], soff, dst);
                else dma16(ru, voff[j], soff, dst);
            }
        };
        f32x16 ag[P::FA][P::FB], au[P::FA][P::FB];
#pragma unroll
        for (int a = 0; a < P::FA; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b) {
                ag[a][b] = f32x16{};
                au[a][b] = f32x16{};
            }
        u32x4 fa[2][P::FA], fg[2][P::FB], fu[2][P::FB];  // [register set][block]
        auto load = [&](const char *st, int s, int buf) {
#pragma unroll
            for (int a = 0; a < P::FA; ++a) fa[buf][a] = frag(st, wm * P::TM + a * 32, s, lane);
#pragma unroll
            for (int b = 0; b < P::FB; ++b) {
                fg[buf][b] = frag(st, BM + wn * P::TN + b * 32, s, lane);
                if constexpr (NB == 2) fu[buf][b] = frag(st, BM + BN + wn * P::TN + b * 32, s, lane);
            }
        };
        auto mma = [&](int buf) {
#pragma unroll
            for (int a = 0; a < P::FA; ++a)
#pragma unroll
                for (int b = 0; b < P::FB; ++b) {
                    ag[a][b] = mfma32(fa[buf][a], fg[buf][b], ag[a][b]);
                    if constexpr (NB == 2) au[a][b] = mfma32(fa[buf][a], fu[buf][b], au[a][b]);
                }
        };
        kloop_pipelined<S, P::NI>(0, KT, smem, P::STAGE, issue, load, mma);
        if constexpr (MODE == kDh) {
            // per 32-row block: every stored g, u is loaded before the first
            // store (one memory round trip per block, not one per row)
#pragma unroll
            for (int a = 0; a < P::FA; ++a) {
                uint16_t gi[16][P::FB], ui[16][P::FB];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = min(m0 + wm * P::TM + a * 32 + mfma32_row(i, lane), rows - 1);
#pragma unroll
                    for (int b = 0; b < P::FB; ++b) {
                        const size_t o = (size_t)r * N + n0 + wn * P::TN + b * 32 + l32;
                        gi[i][b] = g_in[o];
                        ui[i][b] = u_in[o];
                    }
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = m0 + wm * P::TM + a * 32 + mfma32_row(i, lane);
                    if (r >= rows) continue;
#pragma unroll
                    for (int b = 0; b < P::FB; ++b) {
                        const size_t o = (size_t)r * N + n0 + wn * P::TN + b * 32 + l32;
                        const float dh = ag[a][b][i];
                        const float gv = __uint_as_float((uint32_t)gi[i][b] << 16);
                        const float uv = __uint_as_float((uint32_t)ui[i][b] << 16);
                        h[o] = (uint16_t)f32_to_bf16(dh * gv);
                        g_out[o] = (uint16_t)f32_to_bf16(gv > 0.0f ? dh * uv + l1 : 0.0f);
                    }
                }
            }
            __syncthreads();  // the next tile refills the ring
            continue;
        }
#pragma unroll
        for (int a = 0; a < P::FA; ++a)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = m0 + wm * P::TM + a * 32 + mfma32_row(i, lane);
                if (r < rows) {
#pragma unroll
                    for (int b = 0; b < P::FB; ++b) {
                        const size_t o = (size_t)r * N + n0 + wn * P::TN + b * 32 + l32;
                        {
                            const float g = ag[a][b][i] > 0.0f ? ag[a][b][i] : 0.0f;
                            const float u = au[a][b][i];
                            h[o] = (uint16_t)f32_to_bf16(g * u);
                            if constexpr (MODE == kKeep) {
                                if (g_out) g_out[o] = (uint16_t)f32_to_bf16(g);
                                if (u_out) u_out[o] = (uint16_t)f32_to_bf16(u);
                            }
                        }
                    }
                }
            }
        __syncthreads();  // the next tile refills the ring
    }
}

// --------------------------------- down -----------------------------------
template <int BM, int BN, int WM, int WN, int S>
struct DN {
    static constexpr int NW = WM * WN, NTH = NW * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FA = TM / 32, FB = TN / 32;
    static constexpr int BROW = BN * 2;                 // bytes of one W_d row slice
    static constexpr int A_BYTES = BM * kPRow;
    static constexpr int B_BYTES = kPK * BROW;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = S * STAGE;
    static constexpr int NIA = BM / (16 * NW);          // A direct loads per wave and stage
    static constexpr int BR_PER = 1024 / BROW;          // W_d rows per 1 KB direct load
    static constexpr int LPR = BROW / 16;               // lanes (16-byte chunks) per W_d row
    static constexpr int NIB = kPK / BR_PER / NW;       // B direct loads per wave and stage
    static constexpr int NI = NIA + NIB;
    static_assert(BN == 128 || BN == 256, "W_d slice rows of 16 or 32 chunks");
    static_assert(BM % (16 * NW) == 0 && (kPK / BR_PER) % NW == 0, "stage split");
};

// W_d slice rows in a stage: BN / 8 chunks of 16 bytes, chunk c at
// c ^ bsw(row).  A transposing fragment read touches 4 consecutive rows x 4
// chunks in each half-wave; rows 256 or 512 bytes apart start on the same
// bank, and XOR by 4 (row % 4) puts those 16 chunks in 16 different chunk
// positions of one 256-byte bank row, i.e. all 64 banks once.
__device__ __forceinline__ int bsw(int row) { return 4 * (row & 3); }

// Row regions of the unsplit down GEMM's tile grid over the XCDs, by tile
// height.  Its A operand h ([rows][N]) is the larger one (4x W_d at the
// 0.5B and 2B blocks).  With 256-row tiles (the 2B block), 4 row regions x
// 2 column regions (each h row block read by two XCDs) beat the 2 x 4 that
// suit the gate (each read by four): 450.7-453.1 against 467.7-470.3 us,
// cold dense step 1386.5-1387.8 against 1409.4-1410.0 us.  With 128-row
// tiles they cost more than they save on a cold step, when every W_d column
// block then comes from HBM into four XCDs at once: 512.8-516.6 against
// 499.4-500.2 us at the 1B block, 335.5-338.9 against 318.2-318.6 us at the
// paper's block width.
template <int BM>
constexpr int down_rx() { return BM >= 256 ? 4 : 2; }

// PAIRS = 2: y = h W_d + h2 W_d2, the reduction running over the first pair's
// stages, then the second's (same shapes), in one GEMM.
template <int BM, int BN, int WM, int WN, int STG, int PAIRS>
__global__ __launch_bounds__(WM * WN * 64) void down_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ wd, int K, int N,
    const int32_t *__restrict__ rowlist, const int32_t *__restrict__ count, int R_cap,
    float *__restrict__ y, float *__restrict__ partial, const uint16_t *__restrict__ h2,
    const uint16_t *__restrict__ wd2) {
    using P = DN<BM, BN, WM, WN, STG>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int rows = rows_of(count, R_cap);
    const int nrb = (rows + BM - 1) / BM;
    const int ncb = K / BN;
    const int tiles = nrb * ncb;
    const int NS1 = N / kPK;     // stages of one pair's reduction
    const int NS = PAIRS * NS1;  // stages over the whole reduction
    const int S = partial ? split_count(tiles, gridDim.x, NS) : 1;  // reduction splits
    const int work = tiles * S;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31;
    const int g4 = (lane >> 4) & 3, i16 = lane & 15;

    for (int wi = blockIdx.x; wi < work; wi += gridDim.x) {
        // Work items are dealt to the XCDs round-robin (workgroup index % 8).
        // Split-major items (sp = wi % S) give each XCD whole splits: the
        // h and W_d slices of one split, read by all of that split's tiles,
        // then come into one XCD's L2 once.  Tile-major items put one row
        // block on each XCD, and every W_d slice came from beyond the L2
        // once per row block: 40.0 MB fetched per launch at the 0.5B block
        // against 11.7 MB split-major, the size of the operands (same
        // results to the bit: only the workgroup of each item changes).
        const int tile = wi / S, sp = wi % S;
        int rb, cb;
        if (S == 1 && !rowlist) xcd_tile<down_rx<BM>()>(tile, nrb, ncb, rb, cb);
        else { rb = tile % nrb; cb = tile / nrb; }
        const int m0 = rb * BM, k0 = cb * BN;
        const int kt0 = sp * (NS / S), kt1 = kt0 + NS / S;

        const rsrc_t rh = make_rsrc(h + (size_t)m0 * N, (uint64_t)(rows - m0) * N * 2);
        const rsrc_t rd = make_rsrc(wd + k0, ((uint64_t)N * K - k0) * 2);
        const rsrc_t rh2 =
            PAIRS == 2 ? make_rsrc(h2 + (size_t)m0 * N, (uint64_t)(rows - m0) * N * 2) : rh;
        const rsrc_t rd2 = PAIRS == 2 ? make_rsrc(wd2 + k0, ((uint64_t)N * K - k0) * 2) : rd;
        uint32_t aoff[P::NIA], boff[P::NIB];
#pragma unroll
        for (int j = 0; j < P::NIA; ++j) {
            const int row0 = (wave * P::NIA + j) * 16;
            const int r = min(m0 + row0 + (lane >> 2), rows - 1);
            aoff[j] = rows16_voff((uint32_t)(r - m0) * N * 2, lane, row0);
        }
        // B: this lane's W_d row within a 1 KB load and its swizzled chunk
        const int brl = lane / P::LPR;  // 0 .. BR_PER - 1
#pragma unroll
        for (int j = 0; j < P::NIB; ++j) {
            const int row = (wave * P::NIB + j) * P::BR_PER + brl;
            boff[j] = (uint32_t)row * K * 2 + (uint32_t)(((lane % P::LPR) ^ bsw(row)) << 4);
        }
        // one pair's stage kk into ring slot st (each call site passes fixed
        // descriptors: the pair is chosen by a uniform branch, not a select)
        auto put = [&](const rsrc_t ra, const rsrc_t rb, int kk, char *st) {
            const uint32_t soff_a = kk * kPK * 2;
            const uint32_t soff_b = (uint32_t)kk * kPK * K * 2;
#pragma unroll
            for (int j = 0; j < P::NIA; ++j) {
                const int row0 = (wave * P::NIA + j) * 16;
                dma16(ra, aoff[j], soff_a, st + row0 * kPRow);
            }
#pragma unroll
            for (int j = 0; j < P::NIB; ++j) {
                const int row = (wave * P::NIB + j) * P::BR_PER;
                dma16(rb, boff[j], soff_b, st + P::A_BYTES + row * P::BROW);
            }
        };
        auto issue = [&](int kt, char *st) {
            if (PAIRS == 2 && kt >= NS1) put(rh2, rd2, kt - NS1, st);
            else put(rh, rd, kt, st);
        };
        f32x16 acc[P::FA][P::FB];
#pragma unroll
        for (int a = 0; a < P::FA; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b) acc[a][b] = f32x16{};
        u32x4 fa[2][P::FA], fb[2][P::FB];  // [register set][block]
        auto load = [&](const char *st, int s, int buf) {
            const char *bt = st + P::A_BYTES;
#pragma unroll
            for (int a = 0; a < P::FA; ++a) fa[buf][a] = frag(st, wm * P::TM + a * 32, s, lane);
#pragma unroll
            for (int b = 0; b < P::FB; ++b) {
                // lane (g4, i16) supplies row 16 s + 8 (g4 / 2) + 4 hh + i16 / 4,
                // columns c0 + 4 (i16 % 4) ..+3 and receives column c0 + i16
                const int c0 = wn * P::TN + b * 32 + 16 * (g4 & 1) + 4 * (i16 & 3);
                i16x4 v[2];
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int row = 16 * s + 8 * (g4 >> 1) + 4 * hh + (i16 >> 2);
                    const uint32_t off = row * P::BROW + (((c0 >> 3) ^ bsw(row)) << 4) +
                                         (c0 & 7) * 2;
                    v[hh] = lds_tr16((const lds_i16x4 *)(bt + off));
                }
                const u32x2 lo = __builtin_bit_cast(u32x2, v[0]);
                const u32x2 hi = __builtin_bit_cast(u32x2, v[1]);
                fb[buf][b] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        };
        auto mma = [&](int buf) {
#pragma unroll
            for (int a = 0; a < P::FA; ++a)
#pragma unroll
                for (int b = 0; b < P::FB; ++b) acc[a][b] = mfma32(fa[buf][a], fb[buf][b], acc[a][b]);
        };
        kloop_pipelined<STG, P::NI>(kt0, kt1, smem, P::STAGE, issue, load, mma);

        if (S == 1) {
            // per 32-row block: the row indices are all loaded before the
            // first store
#pragma unroll
            for (int a = 0; a < P::FA; ++a) {
                // rows past `rows` read a valid row (clamped) and store nothing
                int yr[16];
                bool ok[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int r = m0 + wm * P::TM + a * 32 + mfma32_row(i, lane);
                    ok[i] = r < rows;
                    const int rr = min(r, rows - 1);
                    yr[i] = rowlist ? rowlist[rr] : rr;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    if (!ok[i]) continue;
#pragma unroll
                    for (int b = 0; b < P::FB; ++b) {
                        y[(size_t)yr[i] * K + k0 + wn * P::TN + b * 32 + l32] = acc[a][b][i];
                    }
                }
            }
        } else {
            // partial tile of split sp, summed in split order later (split_reduce_kernel,
            // or the sparse kernels that take the listed rows; tw_split.hpp).
            // Those read only rows below the count, so rows past it are not
            // stored.
            float *pt = partial + ((size_t)sp * tiles + tile) * (BM * BN);
#pragma unroll
            for (int a = 0; a < P::FA; ++a)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int rl = wm * P::TM + a * 32 + mfma32_row(i, lane);
                    if (m0 + rl >= rows) continue;
#pragma unroll
                    for (int b = 0; b < P::FB; ++b)
                        pt[rl * BN + wn * P::TN + b * 32 + l32] = acc[a][b][i];
                }
        }
        __syncthreads();  // the next work item refills the ring
    }
}

// y[row_r] = sum over splits s = 0, 1, ... of the partial tiles (fixed
// order), when the down GEMM split its reduction.  Each thread owns four
// consecutive outputs (split_sum4).
__global__ __launch_bounds__(256) void split_reduce_kernel(
    const float *__restrict__ partial, const int32_t *__restrict__ rowlist,
    const int32_t *__restrict__ count, int R_cap, int K, int N, float *__restrict__ y) {
    const int rows = rows_of(count, R_cap);
    const int S = split_factor(rows, K, N);
    if (S == 1) return;
    const int K4 = K / 4;
    for (int q = blockIdx.x * 256 + threadIdx.x; q < rows * K4; q += gridDim.x * 256) {
        const int r = q / K4, col = 4 * (q % K4);
        *reinterpret_cast<float4 *>(y + (size_t)(rowlist ? rowlist[r] : r) * K + col) =
            split_sum4(partial, r, col, rows, K, S);
    }
}

// ----------------------- weight gradients of backup rows -------------------
// out[n][k] += sum over r < rows of T[r][n] G[r][k]: a GEMM whose reduction
// runs over the (few) backup slots, so both operands are stored
// reduction-major.  Both land in LDS in their natural row layout (as W_d
// does in the down GEMM) and both fragments are read with the transposing
// ds_read_b64_tr_b16.  T rows past `rows` are clamped to a valid row; G is
// zero-padded to the 32-row stage by gather_rows_kernel, so the last partial
// stage adds exactly zero.
// Tiles of BM (n) x BN (k), both multiples of 128; each operand's stage is
// BM/128 (resp. BN/128) regions of 32 reduction rows x 128 columns (256 B
// rows, chunk c of row r at c ^ bsw(r)), filled by 1 KB direct loads of 4
// rows each.  Three GEMMs (blockIdx.y) share one launch: they have the same
// shape and the tiles of all three fill the chip together.
template <int BM, int BN, int WM, int WN, int S>
struct WGR {
    static constexpr int NW = WM * WN, NTH = NW * 64;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FA = TM / 32, FB = TN / 32;
    static constexpr int REG = kPK * 256;             // one 32 x 128 region
    static constexpr int A_BYTES = BM / 128 * REG, B_BYTES = BN / 128 * REG;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int LDS = S * STAGE;
    static constexpr int LPR = kPK / 4;               // 1 KB loads per region
    static constexpr int NIA = BM / 128 * LPR / NW, NIB = BN / 128 * LPR / NW;
    static constexpr int NI = NIA + NIB;
    static_assert(BM % 128 == 0 && BN % 128 == 0, "128-column regions");
    static_assert((BM / 128 * LPR) % NW == 0 && (BN / 128 * LPR) % NW == 0, "stage split");
    static_assert(TM % 32 == 0 && TN % 32 == 0 && 128 % TN == 0 && 128 % TM == 0,
                  "a wave tile inside one region");
};

// One fragment of a reduction-major region (rows = reduction, 128 columns):
// lane (g4, i16) receives column col32 + 16 (g4 % 2) + i16 at reduction rows
// 16 s + 8 (g4 / 2) .. +7.
__device__ __forceinline__ u32x4 tr_frag(const char *region, int col32, int s, int lane) {
    const int g4 = (lane >> 4) & 3, i16 = lane & 15;
    const int c0 = col32 + 16 * (g4 & 1) + 4 * (i16 & 3);
    i16x4 v[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int row = 16 * s + 8 * (g4 >> 1) + 4 * hh + (i16 >> 2);
        const uint32_t off = row * 256 + (((c0 >> 3) ^ bsw(row)) << 4) + (c0 & 7) * 2;
        v[hh] = lds_tr16((const lds_i16x4 *)(region + off));
    }
    const u32x2 lo = __builtin_bit_cast(u32x2, v[0]);
    const u32x2 hi = __builtin_bit_cast(u32x2, v[1]);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// out_z[n][k] += sum over r < rows of T_z[r][n] G_z[r][k] for z = blockIdx.y
// (T_z [rows][N], G_z [padded rows][K] bf16).  T rows past `rows` are
// clamped to a valid row; G is zero-padded to the 32-row stage by
// gather_rows_kernel, so the last partial stage adds exactly zero.
template <int BM, int BN, int WM, int WN, int STG>
__global__ __launch_bounds__(WM * WN * 64) void wgrad_kernel(
    const uint16_t *__restrict__ T0, const uint16_t *__restrict__ T1,
    const uint16_t *__restrict__ T2, const uint16_t *__restrict__ G0,
    const uint16_t *__restrict__ G1, const uint16_t *__restrict__ G2, int N, int K,
    const int32_t *__restrict__ count, int R_cap, float *__restrict__ out0,
    float *__restrict__ out1, float *__restrict__ out2) {
    using P = WGR<BM, BN, WM, WN, STG>;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int rows = rows_of(count, R_cap);
    if (rows <= 0) return;
    const int z = blockIdx.y;
    const uint16_t *T = z == 0 ? T0 : (z == 1 ? T1 : T2);
    const uint16_t *G = z == 0 ? G0 : (z == 1 ? G1 : G2);
    float *out = z == 0 ? out0 : (z == 1 ? out1 : out2);
    const int NS = (rows + kPK - 1) / kPK;
    const int nrb = N / BM, ncb = K / BN, tiles = nrb * ncb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int l32 = lane & 31;
    const int rl = lane >> 4;  // row within a 1 KB load

    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        int nb, kb;
        xcd_tile(t, nrb, ncb, nb, kb);
        const int n0 = nb * BM, k0 = kb * BN;
        const rsrc_t rt = make_rsrc(T + n0, ((uint64_t)rows * N - n0) * 2);
        const rsrc_t rg = make_rsrc(G + k0, ((uint64_t)NS * kPK * K - k0) * 2);
        auto issue = [&](int kt, char *st) {
#pragma unroll
            for (int j = 0; j < P::NIA; ++j) {
                const int li = wave * P::NIA + j;             // load index in the stage
                const int reg = li / P::LPR, row = (li % P::LPR) * 4;
                const int r = min(kt * kPK + row + rl, rows - 1);
                const uint32_t vo = (uint32_t)r * N * 2 + reg * 256 +
                                    (uint32_t)(((lane & 15) ^ bsw(row + rl)) << 4);
                dma16(rt, vo, 0, st + reg * P::REG + row * 256);
            }
#pragma unroll
            for (int j = 0; j < P::NIB; ++j) {
                const int li = wave * P::NIB + j;
                const int reg = li / P::LPR, row = (li % P::LPR) * 4;
                const uint32_t vo = (uint32_t)(kt * kPK + row + rl) * K * 2 + reg * 256 +
                                    (uint32_t)(((lane & 15) ^ bsw(row + rl)) << 4);
                dma16(rg, vo, 0, st + P::A_BYTES + reg * P::REG + row * 256);
            }
        };
        f32x16 acc[P::FA][P::FB];
#pragma unroll
        for (int a = 0; a < P::FA; ++a)
#pragma unroll
            for (int b = 0; b < P::FB; ++b) acc[a][b] = f32x16{};
        u32x4 fa[2][P::FA], fb[2][P::FB];
        // the wave's columns lie inside one region of each operand
        const int ca = wm * P::TM, cb = wn * P::TN;
        auto load = [&](const char *st, int s, int buf) {
            const char *ra = st + (ca / 128) * P::REG;
            const char *rb = st + P::A_BYTES + (cb / 128) * P::REG;
#pragma unroll
            for (int a = 0; a < P::FA; ++a) fa[buf][a] = tr_frag(ra, ca % 128 + a * 32, s, lane);
#pragma unroll
            for (int b = 0; b < P::FB; ++b) fb[buf][b] = tr_frag(rb, cb % 128 + b * 32, s, lane);
        };
        auto mma = [&](int buf) {
#pragma unroll
            for (int a = 0; a < P::FA; ++a)
#pragma unroll
                for (int b = 0; b < P::FB; ++b) acc[a][b] = mfma32(fa[buf][a], fb[buf][b], acc[a][b]);
        };
        kloop_pipelined<STG, P::NI>(0, NS, smem, P::STAGE, issue, load, mma);
        // add into out: per 32-row block, every old value is loaded before
        // the first store (a store may alias a later load of the same array,
        // so interleaving them would serialise one round trip per element)
#pragma unroll
        for (int a = 0; a < P::FA; ++a) {
            float old[16][P::FB];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int n = n0 + ca + a * 32 + mfma32_row(i, lane);
#pragma unroll
                for (int b = 0; b < P::FB; ++b) old[i][b] = out[(size_t)n * K + k0 + cb + b * 32 + l32];
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int n = n0 + ca + a * 32 + mfma32_row(i, lane);
#pragma unroll
                for (int b = 0; b < P::FB; ++b)
                    out[(size_t)n * K + k0 + cb + b * 32 + l32] = old[i][b] + acc[a][b][i];
            }
        }
        __syncthreads();  // the next tile refills the ring
    }
}

// dst[r] = src[rowlist[r]] (K bf16) for r < rows, zeros for rows <= r <
// rows rounded up to the 32-row stage; one workgroup per slot.
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint16_t *__restrict__ src0, const uint16_t *__restrict__ src1, int K,
    const int32_t *__restrict__ rowlist, const int32_t *__restrict__ count, int R_cap,
    uint16_t *__restrict__ dst0, uint16_t *__restrict__ dst1) {
    const int rows = rows_of(count, R_cap);
    const int r = blockIdx.x;
    const int pad = (rows + kPK - 1) / kPK * kPK;
    if (r >= pad) return;
    const int KC = K >> 3;
    const size_t d = (size_t)r * K;
    if (r < rows) {
        const size_t sidx = (size_t)rowlist[r] * K;
        for (int q = threadIdx.x; q < KC; q += 256) {
            st16(dst0 + d + 8 * q, ld16(src0 + sidx + 8 * q));
            st16(dst1 + d + 8 * q, ld16(src1 + sidx + 8 * q));
        }
    } else {
        for (int q = threadIdx.x; q < KC; q += 256) {
            st16(dst0 + d + 8 * q, u32x4{0u, 0u, 0u, 0u});
            st16(dst1 + d + 8 * q, u32x4{0u, 0u, 0u, 0u});
        }
    }
}

// A kernel instantiation with its shape constants.
template <int BM, int BN, int WM, int WN, int S, int MODE = kGU>
struct GuCfg : GU<BM, BN, WM, WN, S, MODE == kDh ? 1 : 2> {
    static constexpr int BM_ = BM, BN_ = BN;
    static constexpr auto kernel = &gateup_kernel<BM, BN, WM, WN, S, MODE>;
};
template <int BM, int BN, int WM, int WN, int S, int PAIRS = 1>
struct DnCfg : DN<BM, BN, WM, WN, S> {
    static constexpr int BM_ = BM, BN_ = BN;
    static constexpr auto kernel = &down_kernel<BM, BN, WM, WN, S, PAIRS>;
};

// dense comparator shapes and overflow-path shapes (the thin overflow
// tiles do little matrix work per stage, so they keep more stages in flight)
using GuDense = GuCfg<256, 128, 4, 2, 4>;
using GuRows = GuCfg<128, 128, 2, 4, 4>;
// 64 x 64 tiles for all-rows GEMMs too small for 128-row tiles to fill the
// chip: twice the workgroups of 128-column tiles and a quarter of the
// padded rows
using GuSmall = GuCfg<64, 64, 2, 2, 4>;
// row lists of capacity above kTinyRows and at most kSmallRows (the
// inference overflow rows of a batch of thousands): 128 rows x 64 columns of
// g and of u, exactly 256 tiles at 512 rows of capacity; measured 6% faster
// than 64 x 64 tiles at the 0.5B block (16.3 against 17.4 us for ~400
// rows), 64 x 128 was 17.7 us; 8 waves of 32 x 32 (two per SIMD) rather
// than 4 of 64 x 32: 15.1 against 15.7 us at the 0.5B block, 21.6 against
// 23.7 at the paper shape.  A capacity of at most kTinyRows keeps 64 x 64
// tiles: a 128-row tile would stream 128 (repeated) x rows for a handful of
// listed ones, which measured 12.6 us for one row at the 0.5B shape.
constexpr int kTinyRows = 64;
using GuList = GuCfg<128, 64, 4, 2, 4>;
using GuRowsKeep = GuCfg<128, 128, 2, 4, 4, kKeep>;
using GuRowsDh = GuCfg<128, 128, 2, 4, 4, kDh>;
// (the hybrid backup rows' kKeep tiles too: 16.0 against 17.5 us at the
// 0.5B block; the single-operand kDh stage of 192 rows does not split over
// 8 waves and keeps 4)
using GuListKeep = GuCfg<128, 64, 4, 2, 4, kKeep>;
using GuListDh = GuCfg<128, 64, 2, 2, 4, kDh>;
using GuTinyKeep = GuCfg<64, 64, 2, 2, 4, kKeep>;
using GuTinyDh = GuCfg<64, 64, 2, 2, 4, kDh>;

// A row-list gate+up configuration G over a grid of at most grid_cap
// persistent workgroups (sized for the capacity; the rows are counted on the
// device).
template <typename G>
hipError_t launch_gu(int grid_cap, const uint16_t *x, const uint16_t *w1, const uint16_t *w2,
                     int K, int N, const int32_t *rowlist, const int32_t *count, int R_cap,
                     int xrows, uint16_t *o1, uint16_t *o2, uint16_t *o3, const uint16_t *g_in,
                     const uint16_t *u_in, float l1, hipStream_t s,
                     const RowOrder &ord = RowOrder()) {
    hipError_t e = lds_limit_once<G::kernel>(G::LDS);
    if (e != hipSuccess) return e;
    const int tiles = (R_cap + G::BM_ - 1) / G::BM_ * (N / G::BN_);
    const int grid = (tiles < grid_cap ? tiles : grid_cap) + (ord.perm ? row_order_segs(ord.M) : 0);
    hipLaunchKernelGGL(G::kernel, dim3(grid), dim3(G::NTH), G::LDS, s, x, w1, w2, K, N, rowlist,
                       count, R_cap, xrows, o1, o2, o3, g_in, u_in, l1, ord);
    return hipGetLastError();
}
// all rows, 128 x 128 tiles of 8 waves (64 x 32 each, two per SIMD): with
// one tile per CU (the 0.5B block's 256) the 4-wave arrangement leaves a
// single wave per SIMD to wait out every barrier and fragment read; 8 waves
// measured 40.1 against 53-54 us there and the same at two and three tiles
// per CU (paper shape, 1B block)
using DnDense = DnCfg<128, 128, 2, 4, 4>;
// all rows, when its tiles fill the chip: 256 x 256 tiles of 4 waves, one
// per SIMD, each 128 x 128 (its 256 accumulators leave no room for a second
// wave; the 8-wave 64 x 128 arrangement spills), a third fewer LDS bytes per
// flop than 128 x 128 tiles.  Measured at the 2B block: 487 us against 565.
// The same arrangement for the gate+up GEMM (256 accumulators plus two weight
// operands) spilled and measured slower (1053 against 951 us).
using DnBig = DnCfg<256, 256, 2, 2, 4>;
using DnRows = DnCfg<128, 128, 2, 4, 6>;
using DnRowsPair = DnCfg<128, 128, 2, 4, 6, 2>;
static_assert(DnRows::BM_ == kSplitBM && DnRows::BN_ == kSplitBN &&
                  DnRowsPair::BM_ == kSplitBM && DnRowsPair::BN_ == kSplitBN,
              "the split layout of tw_split.hpp");
constexpr int kFillTiles = 256;  // output tiles that fill the chip (one per CU)

using WgCfg = WGR<256, 256, 2, 4, 4>;
constexpr auto kWgrad = &wgrad_kernel<256, 256, 2, 4, 4>;
constexpr auto kWgradSmall = &wgrad_kernel<128, 128, 2, 2, 4>;
using WgSmall = WGR<128, 128, 2, 2, 4>;

}  // namespace

size_t backup_gather_bytes(int R_max, int K) {
    return (size_t)(R_max + kPK - 1) / kPK * kPK * K * 2;
}

hipError_t launch_backup_wgrad(const uint16_t *dy, const uint16_t *x, int K, int N,
                               const int32_t *rowlist, const int32_t *count, int R_cap,
                               const uint16_t *bk_h, const uint16_t *bk_du,
                               const uint16_t *bk_dz, uint16_t *dy_bk, uint16_t *x_bk,
                               float *dwd, float *dwu_t, float *dwg_t, hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    const int pad = (R_cap + kPK - 1) / kPK * kPK;
    hipLaunchKernelGGL(gather_rows_kernel, dim3(pad), dim3(256), 0, s, dy, x, K, rowlist, count,
                       R_cap, dy_bk, x_bk);
    // 256 x 256 tiles (twice the flops per loaded byte of 128 x 128) when
    // they fill the chip, else 128 x 128
    if ((N % 256) == 0 && (K % 256) == 0 && 3 * (N / 256) * (K / 256) >= 128) {
        hipError_t e = lds_limit_once<kWgrad>(WgCfg::LDS);
        if (e != hipSuccess) return e;
        const int tiles = (N / 256) * (K / 256);
        hipLaunchKernelGGL(kWgrad, dim3(tiles < 1024 ? tiles : 1024, 3), dim3(WgCfg::NTH),
                           WgCfg::LDS, s, bk_h, bk_du, bk_dz, dy_bk, x_bk, x_bk, N, K, count,
                           R_cap, dwd, dwu_t, dwg_t);
    } else {
        hipError_t e = lds_limit_once<kWgradSmall>(WgSmall::LDS);
        if (e != hipSuccess) return e;
        const int tiles = (N / 128) * (K / 128);
        hipLaunchKernelGGL(kWgradSmall, dim3(tiles < 1024 ? tiles : 1024, 3), dim3(WgSmall::NTH),
                           WgSmall::LDS, s, bk_h, bk_du, bk_dz, dy_bk, x_bk, x_bk, N, K, count,
                           R_cap, dwd, dwu_t, dwg_t);
    }
    return hipGetLastError();
}

size_t split_partial_bytes() {
    return (size_t)kSplitGrid * DnRows::BM_ * DnRows::BN_ * sizeof(float);
}

hipError_t launch_gateup(const uint16_t *x, int M, const uint16_t *wg_t, const uint16_t *wu_t,
                         int K, int N, const int32_t *rowlist, const int32_t *count, int R_cap,
                         uint16_t *h, hipStream_t s, const RowOrder &ord) {
    if (R_cap <= 0) return hipSuccess;
    constexpr int kAll = 1 << 30;  // no cap: one workgroup per tile
    // the sparse kernel's row order rides on the row-list launches only
    const RowOrder none;
    const RowOrder &o = rowlist ? ord : none;
    // row list: small tiles up to kSmallRows of capacity (the actual count is
    // on the device; overflow rows are a small share of the batch).  All
    // rows: the largest tiles that still fill the chip.
    const bool small = rowlist
                           ? R_cap <= kSmallRows
                           : (R_cap + GuRows::BM_ - 1) / GuRows::BM_ * (N / GuRows::BN_) < kFillTiles;
    if (small && rowlist && R_cap > kTinyRows)
        return launch_gu<GuList>(1024, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h, nullptr,
                                 nullptr, nullptr, nullptr, 0.0f, s, o);
    if (small)
        return launch_gu<GuSmall>(1024, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h, nullptr,
                                  nullptr, nullptr, nullptr, 0.0f, s, o);
    // a row list: one workgroup per CU at most (the grid is sized for the
    // capacity and most of it would find no rows)
    if (rowlist)
        return launch_gu<GuRows>(256, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h, nullptr,
                                 nullptr, nullptr, nullptr, 0.0f, s, o);
    if ((R_cap + GuDense::BM_ - 1) / GuDense::BM_ * (N / GuDense::BN_) >= kFillTiles)
        return launch_gu<GuDense>(kAll, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h, nullptr,
                                  nullptr, nullptr, nullptr, 0.0f, s);
    // all rows, too few 256-row tiles to fill the chip: 128-row tiles
    return launch_gu<GuRows>(kAll, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h, nullptr,
                             nullptr, nullptr, nullptr, 0.0f, s);
}

bool dense_down_split(int M, int K) {
    return ((size_t)M + DnDense::BM_ - 1) / DnDense::BM_ * (size_t)(K / DnDense::BN_) < kFillTiles;
}

hipError_t launch_gateup_keep(const uint16_t *x, int M, const uint16_t *wg_t,
                              const uint16_t *wu_t, int K, int N, const int32_t *rowlist,
                              const int32_t *count, int R_cap, uint16_t *h, uint16_t *g_out,
                              uint16_t *u_out, hipStream_t s) {
    if (!g_out && !u_out) return launch_gateup(x, M, wg_t, wu_t, K, N, rowlist, count, R_cap, h, s);
    if (R_cap <= 0) return hipSuccess;
    // the tiles of launch_gateup's row-list path
    if (R_cap <= kTinyRows)
        return launch_gu<GuTinyKeep>(1024, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h,
                                     g_out, u_out, nullptr, nullptr, 0.0f, s);
    if (R_cap <= kSmallRows)
        return launch_gu<GuListKeep>(1024, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h,
                                     g_out, u_out, nullptr, nullptr, 0.0f, s);
    return launch_gu<GuRowsKeep>(256, x, wg_t, wu_t, K, N, rowlist, count, R_cap, M, h, g_out,
                                 u_out, nullptr, nullptr, 0.0f, s);
}

hipError_t launch_backup_dh(const uint16_t *dy, int M, const uint16_t *wd, int K, int N,
                            const int32_t *rowlist, const int32_t *count, int R_cap,
                            const uint16_t *g_in, const uint16_t *u_in, float l1,
                            uint16_t *du, uint16_t *dz, hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    if (R_cap <= kTinyRows)
        return launch_gu<GuTinyDh>(1024, dy, wd, nullptr, K, N, rowlist, count, R_cap, M, du, dz,
                                   nullptr, g_in, u_in, l1, s);
    if (R_cap <= kSmallRows)
        return launch_gu<GuListDh>(1024, dy, wd, nullptr, K, N, rowlist, count, R_cap, M, du, dz,
                                   nullptr, g_in, u_in, l1, s);
    return launch_gu<GuRowsDh>(256, dy, wd, nullptr, K, N, rowlist, count, R_cap, M, du, dz,
                               nullptr, g_in, u_in, l1, s);
}

hipError_t launch_down(const uint16_t *h, const uint16_t *wd, int K, int N,
                       const int32_t *rowlist, const int32_t *count, int R_cap, float *y,
                       float *partial, hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    if (partial) {
        hipError_t e = lds_limit_once<DnRows::kernel>(DnRows::LDS);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(DnRows::kernel, dim3(kSplitGrid), dim3(DnRows::NTH), DnRows::LDS, s, h,
                           wd, K, N, rowlist, count, R_cap, y, partial, nullptr, nullptr);
    } else if (!rowlist && K % DnBig::BN_ == 0 &&
               (R_cap + DnBig::BM_ - 1) / DnBig::BM_ * (K / DnBig::BN_) >= kFillTiles) {
        hipError_t e = lds_limit_once<DnBig::kernel>(DnBig::LDS);
        if (e != hipSuccess) return e;
        const int tiles = (R_cap + DnBig::BM_ - 1) / DnBig::BM_ * (K / DnBig::BN_);
        hipLaunchKernelGGL(DnBig::kernel, dim3(tiles), dim3(DnBig::NTH), DnBig::LDS, s, h, wd, K,
                           N, rowlist, count, R_cap, y, partial, nullptr, nullptr);
    } else {
        hipError_t e = lds_limit_once<DnDense::kernel>(DnDense::LDS);
        if (e != hipSuccess) return e;
        const int tiles = (R_cap + DnDense::BM_ - 1) / DnDense::BM_ * (K / DnDense::BN_);
        hipLaunchKernelGGL(DnDense::kernel, dim3(tiles), dim3(DnDense::NTH), DnDense::LDS, s, h,
                           wd, K, N, rowlist, count, R_cap, y, partial, nullptr, nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_down_pair(const uint16_t *h, const uint16_t *wd, const uint16_t *h2,
                            const uint16_t *wd2, int K, int N, const int32_t *rowlist,
                            const int32_t *count, int R_cap, float *y, float *partial,
                            hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    hipError_t e = lds_limit_once<DnRowsPair::kernel>(DnRowsPair::LDS);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(DnRowsPair::kernel, dim3(kSplitGrid), dim3(DnRowsPair::NTH),
                       DnRowsPair::LDS, s, h, wd, K, N, rowlist, count, R_cap, y, partial, h2,
                       wd2);
    return hipGetLastError();
}

hipError_t launch_split_reduce(const float *partial, const int32_t *rowlist,
                               const int32_t *count, int R_cap, int K, int N, float *y,
                               hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    // enough workgroups for the largest split case: at most kSplitGrid tiles
    int grid = (int)(((size_t)R_cap * K / 4 + 255) / 256);
    grid = grid < 1024 ? grid : 1024;
    hipLaunchKernelGGL(split_reduce_kernel, dim3(grid), dim3(256), 0, s, partial, rowlist, count,
                       R_cap, K, N, y);
    return hipGetLastError();
}

}  // namespace tw
