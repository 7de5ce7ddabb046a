// hybrid.hip -- hybrid storage of the gate activation for the training
// forward, and the two products that keep it in that form.
//
// Method: "Sparser, Faster, Lighter Transformer Language Models Review",
// section 3-6 (most token rows in a compact ELL-like store of values and
// indices, the few heavy rows whole in a dense backup, a binary routing
// vector per row), section 4-3 (static capacities: at most P stored entries
// per sparse row, a bounded backup, overflow reported for a retry), section
// 2-2 (the training pipeline goes from the TwELL gate to hybrid storage) and
// section 3-7 (dense-to-hybrid and hybrid-to-dense products; in training the
// up and down projections are separate steps that keep the hybrid form).
//
// Kernels
// - hybrid_pack: TwELL -> hybrid.  One wavefront per token row: lane l holds
//   the counts of tiles l, l+64, ...; a wave scan gives each tile's offset
//   in the row's ELL slots, and each lane copies its tiles' entries.  A row
//   whose count exceeds P, or one of whose tiles exceeded the TwELL
//   capacity, is marked in the routing vector instead.
// - route_compact: the ascending list of backup rows from the routing bytes
//   (one workgroup; lane t turns 32 routing bytes into a bit word, then a
//   block scan places the rows), and the true number of backup rows.
// - hybrid_up (sparse rows): u_s = x_m . W_u[:, j_s] for every stored entry,
//   h_s = u_s g_s.  One workgroup of 4 waves per row; entry f goes to wave
//   f % 4; each dot product is a coalesced 1 KB-per-wave gather of the
//   weight row and a DPP wave reduction, four entries in flight per wave.
// - hybrid_down (sparse rows): y_m = sum_s h_s W_d[j_s, :], the down half of
//   the fused inference kernel: the same row split over waves, fp32 partial
//   rows in registers, a fixed-order LDS sum across the 4 waves.
// Backup rows go through the dense MFMA kernels of dense_ffn.hip.
#include "tw_device.hpp"
#include "tw_internal.hpp"

namespace tw {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// ------------------------------- TwELL -> hybrid ---------------------------
__global__ __launch_bounds__(kThreads) void hybrid_pack_kernel(
    const float *__restrict__ tw_val, const int32_t *__restrict__ tw_idx,
    const int32_t *__restrict__ tw_cnt, int M, int NT, int C, int P,
    float *__restrict__ hy_val, int32_t *__restrict__ hy_idx, int32_t *__restrict__ hy_cnt,
    uint8_t *__restrict__ route) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (m >= M) return;  // wave-uniform; no block barrier below

    constexpr int kQ = 4;  // 64-tile chunks: N / T <= 256
    int c[kQ];
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const int t = lane + 64 * q;
        c[q] = t < NT ? tw_cnt[(size_t)m * NT + t] : 0;
    }
    // exclusive offsets of this lane's tiles in the row, the row total, and
    // whether any tile held more than the TwELL capacity
    int off[kQ], base = 0;
    bool over = false;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        int incl = c[q];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        off[q] = base + incl - c[q];
        base += __shfl(incl, 63);
        over |= c[q] > C;
    }
    const int nnz = base;
    const bool heavy = __any(over) || nnz > P;
    if (lane == 0) {
        hy_cnt[m] = nnz;
        route[m] = heavy ? 1 : 0;
    }
    if (heavy) return;
    // every count is <= C and the offsets stay below nnz <= P
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
        const size_t src = ((size_t)m * NT + lane + 64 * q) * C;
        const size_t dst = (size_t)m * P + off[q];
        for (int s = 0; s < c[q]; ++s) {
            hy_idx[dst + s] = tw_idx[src + s];
            hy_val[dst + s] = tw_val[src + s];
        }
    }
}

// --------------------------- routing vector -> list ------------------------
__global__ __launch_bounds__(1024) void route_compact_kernel(
    const uint8_t *__restrict__ route, int M, int R_max, int32_t *__restrict__ bk_rows,
    int32_t *__restrict__ bk_count) {
    __shared__ int s_wsum[16];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int running = 0;
    for (int base = 0; base < M; base += 32 * 1024) {
        const int r0 = base + 32 * tid;  // this thread's 32 rows
        uint32_t word = 0;
        if (r0 + 32 <= M) {
            // 16-byte aligned: route is, and r0 is a multiple of 32
            const u32x4 a = ld16(route + r0), b = ld16(route + r0 + 16);
            const uint32_t v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    word |= (((v[i] >> (8 * k)) & 0xffu) ? 1u : 0u) << (4 * i + k);
        } else {
            for (int i = 0; r0 + i < M && i < 32; ++i) word |= (route[r0 + i] ? 1u : 0u) << i;
        }
        const int cnt = __popc(word);
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int v = __shfl_up(incl, d);
            if (lane >= d) incl += v;
        }
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        int wbase = 0, total = 0;
        for (int q = 0; q < 16; ++q) {
            const int v = s_wsum[q];
            if (q < wave) wbase += v;
            total += v;
        }
        int pos = running + wbase + incl - cnt;
        while (word) {
            const int b = __ffs(word) - 1;
            word &= word - 1u;
            if (pos < R_max) bk_rows[pos] = r0 + b;
            ++pos;
        }
        running += total;
        __syncthreads();  // s_wsum is rewritten by the next chunk
    }
    if (tid == 0) *bk_count = running;
}

// ------------------------ up at the stored entries --------------------------
constexpr int kUpBatch = 4;  // entries gathered together per wave

template <int KCH>
__global__ __launch_bounds__(kThreads) void hybrid_up_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wu_t, int K, int N, int P,
    const float *__restrict__ hy_g, const int32_t *__restrict__ hy_idx,
    const int32_t *__restrict__ hy_cnt, const uint8_t *__restrict__ route,
    float *__restrict__ hy_u, float *__restrict__ hy_h) {
    const int m = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (route[m]) return;  // backup row: the dense path computes it
    const int n = min(hy_cnt[m], P);
    const int ne = (n - wave + kWaves - 1) / kWaves;  // entries f = wave + 4 e of this wave
    if (ne <= 0) return;

    const int KC = K >> 3;  // 16-byte chunks per K-row
    u32x4 xr[KCH];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch) {
        const int q = lane + 64 * ch;
        xr[ch] = q < KC ? ld16(x + (size_t)m * K + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    }
    const size_t row = (size_t)m * P;
    for (int e0 = 0; e0 < ne; e0 += 64) {
        // lane resolves entry e0 + lane
        const int f = wave + kWaves * (e0 + lane);
        int jl = 0;
        float gl = 0.0f, ul = 0.0f;
        if (e0 + lane < ne) {
            // an index outside [0, N) can only come from corrupt storage;
            // clamp it so that the gather stays inside the weights
            jl = min((unsigned)hy_idx[row + f], (unsigned)(N - 1));
            gl = hy_g[row + f];
        }
        const int nb = min(64, ne - e0);
        for (int b = 0; b < nb; b += kUpBatch) {
            int j[kUpBatch];
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u)
                j[u] = __builtin_amdgcn_readlane(jl, b + u < nb ? b + u : b);
            u32x4 wu[kUpBatch][KCH];
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u) {
                const uint16_t *pu = wu_t + (size_t)j[u] * K;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch) {
                    const int q = lane + 64 * ch;
                    wu[u][ch] = q < KC ? ld16(pu + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int u = 0; u < kUpBatch; ++u) {
                float s = 0.0f;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        s += bf_lo(xr[ch][w]) * bf_lo(wu[u][ch][w]);
                        s += bf_hi(xr[ch][w]) * bf_hi(wu[u][ch][w]);
                    }
                s = wave_sum(s);
                if (lane == b + u) ul = s;
            }
        }
        if (e0 + lane < ne) {
            if (hy_u) hy_u[row + f] = ul;
            hy_h[row + f] = ul * gl;
        }
    }
}

// ------------------------- down from the stored entries ---------------------
constexpr int kDnBatch = 4;

template <int KCH>
__global__ __launch_bounds__(kThreads) void hybrid_down_kernel(
    const uint16_t *__restrict__ wd, int K, int N, int P, const float *__restrict__ hy_h,
    const int32_t *__restrict__ hy_idx, const int32_t *__restrict__ hy_cnt,
    const uint8_t *__restrict__ route, float *__restrict__ y) {
    extern __shared__ __attribute__((aligned(16))) char smem[];  // y staging, fp32
    const int m = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (route[m]) return;  // block-uniform: the backup path writes this row
    const int n = min(hy_cnt[m], P);
    const int KC = K >> 3;
    float *yrow = y + (size_t)m * K;
    if (n == 0) {
        for (int q = tid; q < 2 * KC; q += kThreads) st16(yrow + 4 * q, u32x4{0u, 0u, 0u, 0u});
        return;
    }

    float yacc[KCH][8];
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) yacc[ch][e] = 0.0f;

    const size_t row = (size_t)m * P;
    const int ne = (n - wave + kWaves - 1) / kWaves;
    for (int e0 = 0; e0 < ne; e0 += 64) {
        int jl = 0;
        float hl = 0.0f;
        if (e0 + lane < ne) {
            const int f = wave + kWaves * (e0 + lane);
            jl = min((unsigned)hy_idx[row + f], (unsigned)(N - 1));
            hl = hy_h[row + f];
        }
        const int nb = min(64, ne - e0);
        for (int b = 0; b < nb; b += kDnBatch) {
            int j[kDnBatch];
            float h[kDnBatch];
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                const bool ok = b + u < nb;
                const int src = ok ? b + u : b;
                j[u] = __builtin_amdgcn_readlane(jl, src);
                h[u] = ok ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hl), src))
                          : 0.0f;
            }
            u32x4 wv[kDnBatch][KCH];
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u) {
                const uint16_t *pd = wd + (size_t)j[u] * K;
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch) {
                    const int q = lane + 64 * ch;
                    wv[u][ch] = q < KC ? ld16(pd + 8 * q) : u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int u = 0; u < kDnBatch; ++u)
#pragma unroll
                for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        yacc[ch][2 * w] += h[u] * bf_lo(wv[u][ch][w]);
                        yacc[ch][2 * w + 1] += h[u] * bf_hi(wv[u][ch][w]);
                    }
        }
    }

    // y staging, transposed as in the fused inference kernel: element
    // (ch, e) of lane l of wave w at float ((w KCH + ch) 8 + e) 64 + l, so
    // neither the stores nor the loads below have bank conflicts
    float *s_y = reinterpret_cast<float *>(smem);
#pragma unroll
    for (int ch = 0; ch < KCH; ++ch)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_y[((wave * KCH + ch) * 8 + e) * 64 + lane] = yacc[ch][e];
    __syncthreads();
    for (int i = tid; i < 128 * KCH; i += kThreads) {
        const int l = i & 63, half = (i >> 6) & 1, ch = i >> 7;
        const int q = l + 64 * ch;
        if (q >= KC) continue;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int o = (ch * 8 + 4 * half + e) * 64 + l;
            float v = s_y[o];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) v += s_y[(size_t)w * KCH * 512 + o];
            r[e] = v;
        }
        st16(yrow + 8 * q + 4 * half, u32x4{__float_as_uint(r[0]), __float_as_uint(r[1]),
                                            __float_as_uint(r[2]), __float_as_uint(r[3])});
    }
}

template <int KCH>
hipError_t launch_up_k(const uint16_t *x, const uint16_t *wu_t, int M, int K, int N, int P,
                       const float *hy_g, const int32_t *hy_idx, const int32_t *hy_cnt,
                       const uint8_t *route, float *hy_u, float *hy_h, hipStream_t s) {
    hipLaunchKernelGGL(hybrid_up_kernel<KCH>, dim3(M), dim3(kThreads), 0, s, x, wu_t, K, N, P,
                       hy_g, hy_idx, hy_cnt, route, hy_u, hy_h);
    return hipGetLastError();
}

template <int KCH>
hipError_t launch_down_k(const uint16_t *wd, int M, int K, int N, int P, const float *hy_h,
                         const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                         float *y, hipStream_t s) {
    const size_t lds = (size_t)kWaves * KCH * 512 * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&hybrid_down_kernel<KCH>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(hybrid_down_kernel<KCH>, dim3(M), dim3(kThreads), lds, s, wd, K, N, P,
                       hy_h, hy_idx, hy_cnt, route, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_hybrid_pack(const float *tw_val, const int32_t *tw_idx, const int32_t *tw_cnt,
                              int M, int N, int T, int C, int P, float *hy_val, int32_t *hy_idx,
                              int32_t *hy_cnt, uint8_t *route, hipStream_t s) {
    if (M == 0) return hipSuccess;
    hipLaunchKernelGGL(hybrid_pack_kernel, dim3((M + kWaves - 1) / kWaves), dim3(kThreads), 0, s,
                       tw_val, tw_idx, tw_cnt, M, N / T, C, P, hy_val, hy_idx, hy_cnt, route);
    return hipGetLastError();
}

hipError_t launch_route_compact(const uint8_t *route, int M, int R_max, int32_t *bk_rows,
                                int32_t *bk_count, hipStream_t s) {
    hipLaunchKernelGGL(route_compact_kernel, dim3(1), dim3(1024), 0, s, route, M, R_max, bk_rows,
                       bk_count);
    return hipGetLastError();
}

#define TW_KCH_SWITCH(K, CALL)            \
    switch (((K) + 511) / 512) {          \
    case 1: return CALL(1);               \
    case 2: return CALL(2);               \
    case 3: return CALL(3);               \
    case 4: return CALL(4);               \
    case 5: return CALL(5);               \
    case 6: return CALL(6);               \
    case 7: return CALL(7);               \
    default: return CALL(8);              \
    }

hipError_t launch_hybrid_up(const uint16_t *x, const uint16_t *wu_t, int M, int K, int N, int P,
                            const float *hy_g, const int32_t *hy_idx, const int32_t *hy_cnt,
                            const uint8_t *route, float *hy_u, float *hy_h, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define TW_UP(k) launch_up_k<k>(x, wu_t, M, K, N, P, hy_g, hy_idx, hy_cnt, route, hy_u, hy_h, s)
    TW_KCH_SWITCH(K, TW_UP)
#undef TW_UP
}

hipError_t launch_hybrid_down(const uint16_t *wd, int M, int K, int N, int P, const float *hy_h,
                              const int32_t *hy_idx, const int32_t *hy_cnt, const uint8_t *route,
                              float *y, hipStream_t s) {
    if (M == 0) return hipSuccess;
#define TW_DN(k) launch_down_k<k>(wd, M, K, N, P, hy_h, hy_idx, hy_cnt, route, y, s)
    TW_KCH_SWITCH(K, TW_DN)
#undef TW_DN
}

}  // namespace tw
