// dense_ffn.hip -- dense gated FFN on bf16 MFMA: the dense backup of the
// rows that overflow a TwELL tile, and the all-rows dense comparator.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 1-1 equation (h_u = x W_u, h_g = ReLU(x W_g), h = h_u * h_g,
// y = h W_d) and section 3-6 (rows over capacity keep their full activation
// through a dense path on the matrix cores instead of being clipped).
//
// gfx950 design
// - gate+up: one GEMM with two B operands.  Macro tile 256 rows x 128
//   hidden columns, 4 waves in 2 x 2, each wave 128 x 64 outputs of both g
//   and u (2 x 4 x 2 blocks of v_mfma_f32_32x32x16_bf16).  The epilogue forms
//   h = ReLU(g) * u and rounds it to bf16; neither g nor u is stored.
// - down: A = h [rows][N] (reduction-contiguous), B = W_d [N][K] whose
//   reduction index is the row index.  Each thread loads 4 rows x 8 columns
//   of W_d, transposes them in registers and writes them to LDS as 8 rows of
//   4 reduction elements, so the LDS tile has the same swizzled,
//   reduction-contiguous layout as every other operand.  Macro tile 128 x 128.
// - Both kernels take an optional row list (the overflow list) with a
//   device-side count: x rows are gathered through it and y rows scattered
//   through it; workgroups past the count exit at once, so the grid can be
//   sized for the capacity without a host round trip.
#include "tw_device.hpp"
#include "tw_internal.hpp"

namespace tw {
namespace {

constexpr int kThreads = 256;

// ------------------------------ gate + up ---------------------------------
constexpr int kGuBM = 256, kGuBN = 128;
constexpr int kGuA = kGuBM * kRowBytes;  // 32 KB
constexpr int kGuB = kGuBN * kRowBytes;  // 16 KB
constexpr int kGuStage = kGuA + 2 * kGuB;
constexpr int kGuLds = 2 * kGuStage;     // 128 KB

__global__ __launch_bounds__(kThreads) void gateup_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg_t,
    const uint16_t *__restrict__ wu_t, int K, int N, const int32_t *__restrict__ rowlist,
    const int32_t *__restrict__ count, int R_cap, uint16_t *__restrict__ h) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int rows = count ? min(*count, R_cap) : R_cap;
    const int m0 = blockIdx.y * kGuBM;
    if (m0 >= rows) return;
    const int n0 = blockIdx.x * kGuBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r0 = tid >> 3, kc0 = tid & 7;

    int aoff[8], goff[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = min(m0 + r0 + 32 * i, rows - 1);
        const int xr = rowlist ? rowlist[r] : r;
        aoff[i] = xr * K + kc0 * 8;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) goff[i] = (n0 + r0 + 32 * i) * K + kc0 * 8;

    u32x4 ra[8], rg[4], ru[4];
    auto load = [&](int k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ra[i] = ld16(x + aoff[i] + k);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rg[i] = ld16(wg_t + goff[i] + k);
            ru[i] = ld16(wu_t + goff[i] + k);
        }
    };
    auto store = [&](char *st) {
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_st16(st, lds_off(r0 + 32 * i, kc0), ra[i]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lds_st16(st + kGuA, lds_off(r0 + 32 * i, kc0), rg[i]);
            lds_st16(st + kGuA + kGuB, lds_off(r0 + 32 * i, kc0), ru[i]);
        }
    };
    load(0);
    store(smem);
    __syncthreads();

    f32x16 ag[4][2], au[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            ag[a][b] = f32x16{};
            au[a][b] = f32x16{};
        }
    const int KT = K / kBK;
    const int frow = lane & 31;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) load((kt + 1) * kBK);
        const char *st = smem + cur * kGuStage;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int kc = 2 * s + (lane >> 5);
            u32x4 fa[4], fg[2], fu[2];
#pragma unroll
            for (int a = 0; a < 4; ++a) fa[a] = lds_ld16(st, lds_off(wm * 128 + a * 32 + frow, kc));
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                fg[b] = lds_ld16(st + kGuA, lds_off(wn * 64 + b * 32 + frow, kc));
                fu[b] = lds_ld16(st + kGuA + kGuB, lds_off(wn * 64 + b * 32 + frow, kc));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    ag[a][b] = mfma32(fa[a], fg[b], ag[a][b]);
                    au[a][b] = mfma32(fa[a], fu[b], au[a][b]);
                }
        }
        if (more) store(smem + (cur ^ 1) * kGuStage);
        __syncthreads();
    }

    const int l32 = lane & 31;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = m0 + wm * 128 + a * 32 + mfma32_row(i, lane);
            if (r < rows) {
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const float g = ag[a][b][i];
                    const float hv = (g > 0.0f ? g : 0.0f) * au[a][b][i];
                    h[(size_t)r * N + n0 + wn * 64 + b * 32 + l32] = (uint16_t)f32_to_bf16(hv);
                }
            }
        }
}

// --------------------------------- down -----------------------------------
constexpr int kDnBM = 128, kDnBN = 128;
constexpr int kDnA = kDnBM * kRowBytes;  // 16 KB
constexpr int kDnB = kDnBN * kRowBytes;  // 16 KB
constexpr int kDnStage = kDnA + kDnB;
constexpr int kDnLds = 2 * kDnStage;     // 64 KB

__global__ __launch_bounds__(kThreads) void down_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ wd, int K, int N,
    const int32_t *__restrict__ rowlist, const int32_t *__restrict__ count, int R_cap,
    float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int rows = count ? min(*count, R_cap) : R_cap;
    const int m0 = blockIdx.y * kDnBM;
    if (m0 >= rows) return;
    const int k0 = blockIdx.x * kDnBN;  // output columns

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // A (h rows): chunk kc0 of tile rows r0 + 32 i, i < 4
    const int r0 = tid >> 3, kc0 = tid & 7;
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = min(m0 + r0 + 32 * i, rows - 1) * N + kc0 * 8;
    // B (W_d): rows n = 4 nq .. 4 nq + 3 of the stage, columns k0 + 8 ko .. + 7
    const int nq = tid & 15, ko = tid >> 4;
    const int boff = (4 * nq) * K + k0 + 8 * ko;

    u32x4 ra[4], rb[4];
    auto load = [&](int n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = ld16(h + aoff[i] + n);
#pragma unroll
        for (int i = 0; i < 4; ++i) rb[i] = ld16(wd + boff + (n + i) * K);
    };
    auto store = [&](char *st) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lds_st16(st, lds_off(r0 + 32 * i, kc0), ra[i]);
        // transpose 4 (n) x 8 (k) -> 8 LDS rows (k) of 4 reduction elements (n)
        char *sb = st + kDnA;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int w = kk >> 1;
            uint32_t e[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) e[i] = (kk & 1) ? (rb[i][w] >> 16) : (rb[i][w] & 0xffffu);
            const u32x2 v{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
            const int row = 8 * ko + kk;
            *reinterpret_cast<u32x2 *>(sb + lds_off(row, nq >> 1) + (nq & 1) * 8) = v;
        }
    };
    load(0);
    store(smem);
    __syncthreads();

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = f32x16{};
    const int NTK = N / kBK;
    const int frow = lane & 31;
    for (int kt = 0; kt < NTK; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < NTK;
        if (more) load((kt + 1) * kBK);
        const char *st = smem + cur * kDnStage;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int kc = 2 * s + (lane >> 5);
            u32x4 fa[2], fb[2];
#pragma unroll
            for (int a = 0; a < 2; ++a) fa[a] = lds_ld16(st, lds_off(wm * 64 + a * 32 + frow, kc));
#pragma unroll
            for (int b = 0; b < 2; ++b)
                fb[b] = lds_ld16(st + kDnA, lds_off(wn * 64 + b * 32 + frow, kc));
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma32(fa[a], fb[b], acc[a][b]);
        }
        if (more) store(smem + (cur ^ 1) * kDnStage);
        __syncthreads();
    }

    const int l32 = lane & 31;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = m0 + wm * 64 + a * 32 + mfma32_row(i, lane);
            if (r < rows) {
                const int yr = rowlist ? rowlist[r] : r;
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    y[(size_t)yr * K + k0 + wn * 64 + b * 32 + l32] = acc[a][b][i];
            }
        }
}

}  // namespace

hipError_t launch_gateup(const uint16_t *x, const uint16_t *wg_t, const uint16_t *wu_t, int K,
                         int N, const int32_t *rowlist, const int32_t *count, int R_cap,
                         uint16_t *h, hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gateup_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kGuLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(N / kGuBN, (R_cap + kGuBM - 1) / kGuBM);
    hipLaunchKernelGGL(gateup_kernel, grid, dim3(kThreads), kGuLds, s, x, wg_t, wu_t, K, N,
                       rowlist, count, R_cap, h);
    return hipGetLastError();
}

hipError_t launch_down(const uint16_t *h, const uint16_t *wd, int K, int N,
                       const int32_t *rowlist, const int32_t *count, int R_cap, float *y,
                       hipStream_t s) {
    if (R_cap <= 0) return hipSuccess;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&down_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, kDnLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid(K / kDnBN, (R_cap + kDnBM - 1) / kDnBM);
    hipLaunchKernelGGL(down_kernel, grid, dim3(kThreads), kDnLds, s, h, wd, K, N, rowlist,
                       count, R_cap, y);
    return hipGetLastError();
}

}  // namespace tw
