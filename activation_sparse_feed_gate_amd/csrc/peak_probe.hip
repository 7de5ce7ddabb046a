// peak_probe.hip -- achievable peaks of the GPU the kernels run on, printed
// beside the published ones so that roofline fractions can be read against
// both.  A standalone program (not part of libtw.so):
//   - bf16 matrix-core rate: every wave issues long runs of independent
//     v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic), with
//     two waves per SIMD (as the gate GEMM runs) and one;
//   - HBM read rate: a streaming sum over 2 GiB, four 16-byte non-temporal
//     loads in flight per lane;
//   - HBM copy rate: the same stream copied to a second 2 GiB buffer;
//   - how the matrix-core rate depends on the operand values: the register
//     loop again with pseudo-random bf16 operands, and the gate GEMM's own
//     main loop (tw_gemm.hpp: 256 x 256 tiles, 8 waves, the direct-to-LDS
//     ring; no epilogue) at the 0.5B and 2B block shapes on all-zero,
//     constant and pseudo-random operands.  The part lowers its clock under
//     the power that toggling multiplier inputs draw, so the same
//     instructions run at different rates on different data.
// Each of the first four figures is the best of a few repetitions (the first
// launches run while the clocks ramp up); the main-loop figures are the
// median of ten launches after four warm-up ones.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include <algorithm>
#include <vector>

#include "tw_device.hpp"
#include "tw_gemm.hpp"

namespace {

using tw::f32x16;
using tw::u32x4;
typedef float f4 __attribute__((ext_vector_type(4)));

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void mfma_loop(float *out, int iters) {
    const int lane = threadIdx.x & 63;
    const u32x4 a = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, (uint32_t)lane};
    const u32x4 b = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = tw::mfma32(a, b, acc[i]);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the products live
}

// A pseudo-random bf16 pair in [-1, 1) (magnitudes 2^-4 .. 1, random sign
// and mantissa) from a 32-bit hash of (seed, index).
__host__ __device__ inline uint32_t hash32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}
__host__ __device__ inline uint16_t rand_bf16(uint32_t r) {
    return (uint16_t)(((r >> 15) & 1u) << 15 | (0x7bu + (r & 3u)) << 7 | ((r >> 2) & 0x7fu));
}
__host__ __device__ inline uint32_t rand_pair(uint32_t seed, uint32_t i) {
    const uint32_t r = hash32(seed * 0x9e3779b9u + i);
    return (uint32_t)rand_bf16(r) | (uint32_t)rand_bf16(hash32(r)) << 16;
}

// The register loop on pseudo-random operands: four A and four B fragments
// per lane, so consecutive matrix instructions read different values.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void mfma_loop_rand(float *out, int iters) {
    const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[j][e] = rand_pair(g, 8 * j + e);
            b[j][e] = rand_pair(g, 8 * j + 4 + e);
        }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = tw::mfma32(a[i & 3], b[(i + (i >> 2)) & 3], acc[i]);
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The gate GEMM's main loop alone: A [M][K] and B [N][K] bf16, 256 x 256
// output tiles on 8 waves (4 x 2, 64 x 128 each, v_mfma_f32_32x32x16_bf16),
// operands streamed through the 4-stage direct-to-LDS ring of tw_gemm.hpp,
// tiles mapped to the XCDs as the gate maps them.  Each thread writes the sum
// of its accumulators (keeping the products live); M and N are multiples
// of 256.
constexpr int kLoopBM = 256;
constexpr int kLoopStage = 2 * kLoopBM * tw::kPRow;  // 32 KB
constexpr int kLoopStages = 4;

__global__ __launch_bounds__(512) void gate_main_loop(const uint16_t *__restrict__ A,
                                                      const uint16_t *__restrict__ B, int M,
                                                      int N, int K, float *__restrict__ out) {
    using namespace tw;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int bm, bn;
    xcd_tile(blockIdx.x, M / kLoopBM, N / kLoopBM, bm, bn);
    const int m0 = bm * kLoopBM, n0 = bn * kLoopBM;
    const rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint64_t)kLoopBM * K * 2);
    const rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint64_t)kLoopBM * K * 2);
    uint32_t aoff[2], boff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row0 = wave * 32 + j * 16;
        const uint32_t r = (uint32_t)(row0 + (lane >> 2));
        aoff[j] = rows16_voff(r * K * 2, lane, row0);
        boff[j] = rows16_voff(r * K * 2, lane, row0);
    }
    auto issue = [&](int kt, char *st) {
        const uint32_t soff = kt * kPK * 2;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row0 = wave * 32 + j * 16;
            dma16(ra, aoff[j], soff, st + row0 * kPRow);
            dma16(rb, boff[j], soff, st + (kLoopBM + row0) * kPRow);
        }
    };
    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x16{};
    u32x4 fa[2][2], fb[2][4];
    auto load = [&](const char *st, int s, int buf) {
        const char *bt = st + kLoopBM * kPRow;
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
    settle_scalars(out);
    kloop_pipelined<kLoopStages, 4>(0, K / kPK, smem, kLoopStage, issue, load, mma);
    float v = 0.f;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) v += acc[a][b][i];
    out[(size_t)blockIdx.x * 512 + tid] = v;
}

// lane-strided stream over n 16-byte elements, four loads in flight per lane
__global__ __launch_bounds__(256) void read_stream(const f4 *__restrict__ src, float *__restrict__ out,
                                                   size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
        f4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t k = i + u * stride;
            v[u] = k < n ? __builtin_nontemporal_load(src + k) : f4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc += v[u];
    }
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc.x + acc.y + acc.z + acc.w;
}

__global__ __launch_bounds__(256) void copy_stream(const f4 *__restrict__ src, f4 *__restrict__ dst,
                                                   size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += 4 * stride) {
        f4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t k = i + u * stride;
            if (k < n) v[u] = __builtin_nontemporal_load(src + k);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t k = i + u * stride;
            if (k < n) __builtin_nontemporal_store(v[u], dst + k);
        }
    }
}

#define CHECK(x)                                                                          \
    do {                                                                                  \
        const hipError_t e_ = (x);                                                        \
        if (e_ != hipSuccess) {                                                           \
            std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                  \
            return 1;                                                                     \
        }                                                                                 \
    } while (0)

}  // namespace

int main() {
    constexpr double kPeakBf16 = 2516.6;  // TFLOP/s, dense (256 CUs x 4096 flop/clk x 2.4 GHz)
    constexpr double kPeakHbm = 8000.0;   // GB/s
    constexpr int kGrid = 256 * 4;        // four workgroups per CU
    constexpr int kIters = 4096;
    constexpr int kStreamGrid = 256 * 32;
    constexpr size_t kBytes = (size_t)2 << 30;
    constexpr size_t kN = kBytes / 16;

    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    float *out = nullptr, *sums = nullptr;
    f4 *src = nullptr, *dst = nullptr;
    CHECK(hipMalloc(&out, (size_t)kGrid * 512 * sizeof(float)));         // mfma_loop<8>: 512 lanes
    CHECK(hipMalloc(&sums, (size_t)kStreamGrid * 256 * sizeof(float)));  // read_stream: one per lane
    CHECK(hipMalloc(&src, kBytes));
    CHECK(hipMalloc(&dst, kBytes));
    CHECK(hipMemset(src, 0, kBytes));
    CHECK(hipMemset(dst, 0, kBytes));

    auto timed = [&](auto launch, float &best_ms) -> hipError_t {
        best_ms = 1e30f;
        for (int rep = 0; rep < 5; ++rep) {
            hipError_t e = hipEventRecord(e0);
            if (e != hipSuccess) return e;
            launch();
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if ((e = hipEventRecord(e1)) != hipSuccess) return e;
            if ((e = hipEventSynchronize(e1)) != hipSuccess) return e;
            float ms = 0.0f;
            if ((e = hipEventElapsedTime(&ms, e0, e1)) != hipSuccess) return e;
            if (ms < best_ms) best_ms = ms;
        }
        return hipSuccess;
    };

    float ms = 0.0f;
    const double mfma_flop = 32.0 * 32 * 16 * 2;
    CHECK(timed([&] { hipLaunchKernelGGL(mfma_loop<8>, dim3(kGrid), dim3(512), 0, 0, out, kIters); }, ms));
    double tf = (double)kGrid * 8 * kIters * 8 * mfma_flop / ms / 1e9;
    std::printf("bf16 MFMA, 2 waves per SIMD: %.1f TFLOP/s (%.1f%% of %.1f)\n", tf, 100 * tf / kPeakBf16,
                kPeakBf16);
    CHECK(timed([&] { hipLaunchKernelGGL(mfma_loop<4>, dim3(kGrid), dim3(256), 0, 0, out, kIters); }, ms));
    tf = (double)kGrid * 4 * kIters * 8 * mfma_flop / ms / 1e9;
    std::printf("bf16 MFMA, 1 wave per SIMD: %.1f TFLOP/s (%.1f%% of %.1f)\n", tf, 100 * tf / kPeakBf16,
                kPeakBf16);
    CHECK(timed([&] { hipLaunchKernelGGL(read_stream, dim3(kStreamGrid), dim3(256), 0, 0, src, sums, kN); },
                ms));
    double gbs = kBytes / ms / 1e6;
    std::printf("HBM read, 2 GiB: %.0f GB/s (%.1f%% of %.0f)\n", gbs, 100 * gbs / kPeakHbm, kPeakHbm);
    CHECK(timed([&] { hipLaunchKernelGGL(copy_stream, dim3(kStreamGrid), dim3(256), 0, 0, src, dst, kN); },
                ms));
    gbs = 2.0 * kBytes / ms / 1e6;
    std::printf("HBM copy, 2 GiB read + 2 GiB written: %.0f GB/s (%.1f%% of %.0f)\n", gbs,
                100 * gbs / kPeakHbm, kPeakHbm);

    CHECK(hipFree(dst));
    CHECK(hipFree(src));
    CHECK(hipFree(sums));

    CHECK(timed([&] { hipLaunchKernelGGL(mfma_loop_rand<8>, dim3(kGrid), dim3(512), 0, 0, out, kIters); },
                ms));
    tf = (double)kGrid * 8 * kIters * 8 * mfma_flop / ms / 1e9;
    std::printf("bf16 MFMA, 2 waves per SIMD, pseudo-random operands: %.1f TFLOP/s (%.1f%% of %.1f)\n",
                tf, 100 * tf / kPeakBf16, kPeakBf16);
    CHECK(hipFree(out));

    // the gate's main loop at the 0.5B and 2B block shapes, by operand values
    CHECK(hipFuncSetAttribute(reinterpret_cast<const void *>(gate_main_loop),
                              hipFuncAttributeMaxDynamicSharedMemorySize,
                              kLoopStages * kLoopStage));
    struct Shape { const char *name; int M, N, K; };
    const Shape shapes[] = {{"0.5B block, 4096 x 4096 x 1024", 4096, 4096, 1024},
                            {"2B block, 16384 x 8192 x 2048", 16384, 8192, 2048}};
    for (const Shape &sh : shapes) {
        const size_t na = (size_t)sh.M * sh.K, nb = (size_t)sh.N * sh.K;
        const int tiles = (sh.M / kLoopBM) * (sh.N / kLoopBM);
        uint16_t *A = nullptr, *B = nullptr;
        float *o = nullptr;
        CHECK(hipMalloc(&A, na * 2));
        CHECK(hipMalloc(&B, nb * 2));
        CHECK(hipMalloc(&o, (size_t)tiles * 512 * sizeof(float)));
        const char *fills[] = {"all-zero", "constant (0.0115)", "pseudo-random"};
        for (int f = 0; f < 3; ++f) {
            if (f < 2) {
                CHECK(hipMemset(A, f ? 0x3c : 0, na * 2));
                CHECK(hipMemset(B, f ? 0x3c : 0, nb * 2));
            } else {
                std::vector<uint16_t> h(na > nb ? na : nb);
                for (size_t i = 0; i < na; ++i) h[i] = rand_bf16(hash32((uint32_t)i * 2u + 1u));
                CHECK(hipMemcpy(A, h.data(), na * 2, hipMemcpyHostToDevice));
                for (size_t i = 0; i < nb; ++i) h[i] = rand_bf16(hash32((uint32_t)i * 2u + 2u));
                CHECK(hipMemcpy(B, h.data(), nb * 2, hipMemcpyHostToDevice));
            }
            std::vector<float> t;
            for (int rep = 0; rep < 14; ++rep) {
                CHECK(hipEventRecord(e0));
                hipLaunchKernelGGL(gate_main_loop, dim3(tiles), dim3(512), kLoopStages * kLoopStage,
                                   0, A, B, sh.M, sh.N, sh.K, o);
                CHECK(hipGetLastError());
                CHECK(hipEventRecord(e1));
                CHECK(hipEventSynchronize(e1));
                CHECK(hipEventElapsedTime(&ms, e0, e1));
                if (rep >= 4) t.push_back(ms);
            }
            std::sort(t.begin(), t.end());
            const double med = t[t.size() / 2];
            tf = 2.0 * sh.M * sh.N * sh.K / med / 1e9;
            std::printf("gate main loop, %s, %s operands: %.1f us (min %.1f, max %.1f), %.1f TFLOP/s "
                        "(%.1f%% of %.1f)\n",
                        sh.name, fills[f], med * 1e3, t.front() * 1e3, t.back() * 1e3, tf,
                        100 * tf / kPeakBf16, kPeakBf16);
        }
        CHECK(hipFree(o));
        CHECK(hipFree(B));
        CHECK(hipFree(A));
    }
    return 0;
}
