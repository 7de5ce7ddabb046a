// peak_probe.hip -- achievable peaks of the GPU the kernels run on, printed
// beside the published ones so that roofline fractions can be read against
// both.  A standalone program (not part of libtw.so):
//   - bf16 matrix-core rate: every wave issues long runs of independent
//     v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic), with
//     two waves per SIMD (as the gate GEMM runs) and one;
//   - HBM read rate: a streaming sum over 2 GiB, four 16-byte non-temporal
//     loads in flight per lane;
//   - HBM copy rate: the same stream copied to a second 2 GiB buffer.
// Each figure is the best of a few repetitions (the first launches run
// while the clocks ramp up).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "tw_device.hpp"

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
    CHECK(hipFree(out));
    return 0;
}
