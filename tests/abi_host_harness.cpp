// Host-only harness over the C ABI's argument validation (include/tw.h),
// built with AddressSanitizer and UndefinedBehaviorSanitizer on the host
// side by tests/test_sanitizers.py and run on the CPU.
//
// Every call below must be rejected on the host before anything reaches a
// device: the pointers are fake (aligned or misaligned addresses that are
// never dereferenced), and the sizes include the extremes of int so that an
// overflowing size computation in the validation or in a workspace query
// is caught by the sanitizer.  Prints HARNESS_OK and exits 0 when every
// status is the expected one.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "tw.h"

namespace {

int g_fail = 0;

#define EXPECT(call, want)                                                               \
    do {                                                                                 \
        const int got_ = (int)(call);                                                    \
        if (got_ != (want)) {                                                            \
            std::printf("FAIL line %d: %s -> %d, want %d (%s)\n", __LINE__, #call, got_,  \
                        (want), tw_last_error());                                        \
            ++g_fail;                                                                    \
        } else if (got_ != TW_OK && std::strlen(tw_last_error()) == 0) {                 \
            std::printf("FAIL line %d: %s gave no message\n", __LINE__, #call);         \
            ++g_fail;                                                                    \
        }                                                                                \
    } while (0)

#define EXPECT_ZERO(expr)                                                               \
    do {                                                                                \
        const size_t v_ = (expr);                                                       \
        if (v_ != 0) {                                                                  \
            std::printf("FAIL line %d: %s -> %zu, want 0\n", __LINE__, #expr, v_);      \
            ++g_fail;                                                                   \
        }                                                                               \
    } while (0)

template <typename T>
T *fake(uintptr_t a) {
    return reinterpret_cast<T *>(a);
}

const uintptr_t A = 0x100000;  // 16-byte aligned, never dereferenced

tw_status pack(int M, int K, int N, int T, int C, int R, size_t ws = 1 << 20,
               uintptr_t x = A, uintptr_t val = A, uintptr_t z = 0) {
    return tw_pack_gate(fake<uint16_t>(x), fake<uint16_t>(A), M, K, N, T, C, fake<float>(val),
                        fake<int32_t>(A), fake<int32_t>(A), fake<int32_t>(A), fake<int32_t>(A),
                        R, fake<float>(z), fake<void>(A), ws, nullptr, nullptr);
}

tw_status sparse(int M, int K, int N, int T, int C, int R, size_t ws = 1 << 20, uintptr_t y = A) {
    return tw_sparse_ffn_fwd(fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A),
                             fake<uint16_t>(A), M, K, N, T, C, fake<float>(A), fake<int32_t>(A),
                             fake<int32_t>(A), fake<int32_t>(A), fake<int32_t>(A), R,
                             fake<float>(y), fake<void>(A), ws, nullptr, nullptr);
}

tw_status hpack(int M, int N, int T, int C, int P, int R) {
    return tw_hybrid_pack(M, N, T, C, fake<float>(A), fake<int32_t>(A), fake<int32_t>(A), P,
                          fake<float>(A), fake<int32_t>(A), fake<int32_t>(A), fake<uint8_t>(A),
                          fake<int32_t>(A), fake<int32_t>(A), R, nullptr, nullptr);
}

tw_status hup(int M, int K, int N, int P, int R) {
    return tw_hybrid_up(fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A), M, K, N, P,
                        fake<float>(A), fake<int32_t>(A), fake<int32_t>(A), fake<uint8_t>(A),
                        fake<int32_t>(A), fake<int32_t>(A), R, nullptr, fake<float>(A), nullptr,
                        nullptr, fake<uint16_t>(A), nullptr, nullptr);
}

tw_status hdown(int M, int K, int N, int P, int R, size_t ws) {
    return tw_hybrid_down(fake<uint16_t>(A), M, K, N, P, fake<float>(A), fake<int32_t>(A),
                          fake<int32_t>(A), fake<uint8_t>(A), fake<int32_t>(A), fake<int32_t>(A),
                          R, fake<uint16_t>(A), fake<float>(A), fake<void>(A), ws, nullptr,
                          nullptr);
}

tw_status bdh(int M, int K, int N, int P, int R, uintptr_t du = A) {
    return tw_hybrid_bwd_dh(fake<uint16_t>(A), fake<uint16_t>(A), M, K, N, P, 0.01f,
                            fake<float>(A), fake<float>(A), fake<int32_t>(A), fake<int32_t>(A),
                            fake<uint8_t>(A), fake<int32_t>(A), fake<int32_t>(A), R,
                            fake<uint16_t>(A), fake<uint16_t>(A), fake<float>(du), fake<float>(A),
                            fake<uint16_t>(A), fake<uint16_t>(A), nullptr, nullptr);
}

tw_status bdx(int M, int K, int N, int P, int R, size_t ws) {
    return tw_hybrid_bwd_dx(fake<uint16_t>(A), fake<uint16_t>(A), M, K, N, P, fake<float>(A),
                            fake<float>(A), fake<int32_t>(A), fake<int32_t>(A), fake<uint8_t>(A),
                            fake<int32_t>(A), fake<int32_t>(A), R, fake<uint16_t>(A),
                            fake<uint16_t>(A), fake<float>(A), fake<void>(A), ws, nullptr,
                            nullptr);
}

tw_status bdw(int M, int K, int N, int P, int R, size_t ws) {
    return tw_hybrid_bwd_dw(fake<uint16_t>(A), fake<uint16_t>(A), M, K, N, P, fake<float>(A),
                            fake<float>(A), fake<float>(A), fake<int32_t>(A), fake<int32_t>(A),
                            fake<uint8_t>(A), fake<int32_t>(A), fake<int32_t>(A), R,
                            fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A),
                            fake<float>(A), fake<float>(A), fake<float>(A), fake<void>(A), ws,
                            nullptr, nullptr);
}

}  // namespace

int main() {
    // status strings, including values outside the enum
    EXPECT(std::strcmp(tw_status_str(TW_OK), "TW_OK"), 0);
    EXPECT(std::strcmp(tw_status_str(-7), "TW_UNKNOWN"), 0);
    EXPECT(std::strcmp(tw_status_str(INT_MAX), "TW_UNKNOWN"), 0);

    // workspace queries: zero for every rejected shape, including the int extremes
    EXPECT_ZERO(tw_workspace_bytes(INT_MAX, 4096, 8192, 128, 8, 0));
    EXPECT_ZERO(tw_workspace_bytes(INT_MIN, 1024, 4096, 128, 8, 0));
    EXPECT_ZERO(tw_workspace_bytes(4096, INT_MAX, 4096, 128, 8, 512));
    EXPECT_ZERO(tw_workspace_bytes(4096, 1024, INT_MAX, 128, 8, 512));
    EXPECT_ZERO(tw_workspace_bytes(4096, 1024, 4096, INT_MAX, 8, 512));
    EXPECT_ZERO(tw_workspace_bytes(4096, 1024, 4096, 128, INT_MAX, 512));
    EXPECT_ZERO(tw_workspace_bytes(4096, 1024, 4096, 128, 8, INT_MAX));
    EXPECT_ZERO(tw_workspace_bytes(4096, 1024, 4096, 128, 8, -1));
    if (tw_workspace_bytes(4096, 1024, 4096, 128, 8, 512) == 0) {
        std::printf("FAIL: valid shape gave no workspace\n");
        ++g_fail;
    }
    // the largest accepted shapes give a size, not an overflow
    (void)tw_workspace_bytes(524287, 4096, 65536, 256, 256, 524287);
    (void)tw_ffn_workspace_bytes(524287, 4096, 65536);
    (void)tw_ffn_workspace_bytes(INT_MAX, INT_MAX, INT_MAX);
    (void)tw_pack_dense_workspace_bytes(INT_MAX, INT_MAX);
    (void)tw_hybrid_down_workspace_bytes(INT_MAX);
    (void)tw_hybrid_bwd_dx_workspace_bytes(INT_MAX);
    (void)tw_hybrid_bwd_dw_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX);
    (void)tw_hybrid_bwd_dw_workspace_bytes(-1, -1, -1, -1, -1);

    // tw_pack_gate
    EXPECT(pack(64, 256, 1024, 64, 8, 64), TW_EUNSUPPORTED);          // T
    EXPECT(pack(64, 256, 1000, 128, 8, 64), TW_EINVAL);               // N % T
    EXPECT(pack(64, 256, 1024, 128, 0, 64), TW_EINVAL);               // C
    EXPECT(pack(64, 256, 1024, 128, 129, 64), TW_EINVAL);
    EXPECT(pack(64, 192, 1024, 128, 8, 64), TW_EUNSUPPORTED);         // K % 128
    EXPECT(pack(64, 8192, 1024, 128, 8, 64), TW_EUNSUPPORTED);        // K > 4096
    EXPECT(pack(64, 256, 1024, 128, 8, 65), TW_EINVAL);               // R_max > M
    EXPECT(pack(-1, 256, 1024, 128, 8, 0), TW_EINVAL);
    EXPECT(pack(INT_MIN, 256, 1024, 128, 8, 0), TW_EINVAL);
    EXPECT(pack(INT_MAX, 4096, 1024, 128, 8, 0), TW_EUNSUPPORTED);    // x over 4 GiB
    EXPECT(pack(64, INT_MAX, 1024, 128, 8, 64), TW_EUNSUPPORTED);
    EXPECT(pack(64, 256, INT_MAX, 128, 8, 64), TW_EINVAL);
    EXPECT(pack(64, 256, 128 * 300, 128, 8, 64), TW_EUNSUPPORTED);    // N / T > 256
    EXPECT(pack(64, 256, 1024, 128, 8, 64, 16), TW_EINVAL);           // workspace too small
    EXPECT(pack(64, 256, 1024, 128, 8, 64, 1 << 20, 0), TW_EINVAL);   // x NULL
    EXPECT(pack(64, 256, 1024, 128, 8, 64, 1 << 20, A + 8), TW_EINVAL);
    EXPECT(pack(64, 256, 1024, 128, 8, 64, 1 << 20, A, A + 4), TW_EINVAL);
    EXPECT(pack(64, 256, 1024, 128, 8, 64, 1 << 20, A, A, A + 4), TW_EINVAL);  // z_debug

    // tw_gate_dense / tw_pack_dense
    EXPECT(tw_gate_dense(fake<uint16_t>(A), fake<uint16_t>(A), 64, 100, 1024, fake<float>(A),
                         nullptr, nullptr), TW_EUNSUPPORTED);
    EXPECT(tw_gate_dense(nullptr, fake<uint16_t>(A), 64, 256, 1024, fake<float>(A), nullptr,
                         nullptr), TW_EINVAL);
    EXPECT(tw_gate_dense(fake<uint16_t>(A), fake<uint16_t>(A), INT_MAX, 256, 1024, fake<float>(A),
                         nullptr, nullptr), TW_EUNSUPPORTED);
    EXPECT(tw_gate_dense(fake<uint16_t>(A), fake<uint16_t>(A), 64, 8192, 1024, fake<float>(A),
                         nullptr, nullptr), TW_EUNSUPPORTED);
    EXPECT(tw_pack_dense(fake<float>(A), 64, 1024, 128, 8, fake<float>(A), fake<int32_t>(A),
                         fake<int32_t>(A), fake<int32_t>(A), fake<int32_t>(A), 64, fake<void>(A),
                         8, nullptr, nullptr), TW_EINVAL);
    EXPECT(tw_pack_dense(fake<float>(A), INT_MAX, INT_MAX, 128, 8, fake<float>(A),
                         fake<int32_t>(A), fake<int32_t>(A), fake<int32_t>(A), fake<int32_t>(A),
                         0, fake<void>(A), 1 << 20, nullptr, nullptr) == TW_OK ? -1 : 0, 0);

    // tw_sparse_ffn_fwd / tw_ffn_fwd
    EXPECT(sparse(64, 256, 1024, 128, 16, 64, 1 << 20, 0), TW_EINVAL);  // y NULL
    EXPECT(sparse(64, 256, 1024, 100, 16, 64), TW_EUNSUPPORTED);
    EXPECT(sparse(64, 256, 1024, 128, 16, 64, 8), TW_EINVAL);
    EXPECT(sparse(INT_MAX, 256, 1024, 128, 16, INT_MAX), TW_EUNSUPPORTED);
    EXPECT(tw_ffn_fwd(fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A),
                      64, 256, 1000, fake<float>(A), fake<void>(A), 1 << 24, nullptr, nullptr),
           TW_EUNSUPPORTED);
    EXPECT(tw_ffn_fwd(fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A), nullptr, 64, 256,
                      1024, fake<float>(A), fake<void>(A), 1 << 24, nullptr, nullptr), TW_EINVAL);
    EXPECT(tw_ffn_fwd(fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A),
                      64, 4096, 1 << 19, fake<float>(A), fake<void>(A), SIZE_MAX, nullptr,
                      nullptr), TW_EUNSUPPORTED);
    EXPECT(tw_ffn_fwd(fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A), fake<uint16_t>(A),
                      INT_MAX, INT_MAX, INT_MAX, fake<float>(A), fake<void>(A), SIZE_MAX, nullptr,
                      nullptr) == TW_OK ? -1 : 0, 0);

    // hybrid forward
    EXPECT(hpack(64, 1024, 128, 16, 0, 8), TW_EINVAL);
    EXPECT(hpack(64, 1024, 128, 16, 1025, 8), TW_EINVAL);
    EXPECT(hpack(64, 1024, 64, 16, 128, 8), TW_EUNSUPPORTED);
    EXPECT(hpack(1 << 17, 1 << 15, 128, 16, 128, 1 << 17), TW_EUNSUPPORTED);
    EXPECT(hpack(1 << 20, 4096, 128, 16, 4096, 0), TW_EUNSUPPORTED);   // M * P slot ids
    EXPECT(hpack(INT_MAX, 4096, 128, 16, INT_MAX, INT_MAX), TW_EUNSUPPORTED);
    EXPECT(hup(64, 100, 1024, 128, 8), TW_EUNSUPPORTED);
    EXPECT(hup(1 << 20, 256, 4096, 4096, 0), TW_EUNSUPPORTED);
    EXPECT(hup(64, 256, 1024, 0, 8), TW_EINVAL);
    const size_t nws = tw_hybrid_down_workspace_bytes(8);
    EXPECT(hdown(64, 256, 1024, 128, 8, nws - 1), TW_EINVAL);
    EXPECT(hdown(64, 256, 1024, 2048, 8, nws), TW_EINVAL);
    EXPECT(hdown(1 << 20, 256, 4096, 4096, 0, 0), TW_EUNSUPPORTED);

    // hybrid backward
    EXPECT(bdh(64, 100, 1024, 128, 8), TW_EUNSUPPORTED);
    EXPECT(bdh(64, 256, 1024, 128, 65), TW_EINVAL);
    EXPECT(bdh(64, 256, 1024, 128, 8, 0), TW_EINVAL);
    EXPECT(bdh(64, 256, 1024, 128, 8, A + 4), TW_EINVAL);
    EXPECT(bdh(1 << 20, 256, 4096, 4096, 0), TW_EUNSUPPORTED);
    const size_t nx = tw_hybrid_bwd_dx_workspace_bytes(8);
    EXPECT(bdx(64, 256, 1024, 128, 8, nx - 1), TW_EINVAL);
    EXPECT(bdx(1 << 20, 256, 4096, 4096, 0, 0), TW_EUNSUPPORTED);
    const size_t nw = tw_hybrid_bwd_dw_workspace_bytes(64, 256, 1024, 128, 8);
    EXPECT(bdw(64, 256, 1024, 128, 8, nw - 1), TW_EINVAL);
    EXPECT(bdw(64, 256, 1024, 2048, 8, nw), TW_EINVAL);
    EXPECT(bdw(1 << 20, 256, 1 << 15, 1 << 12, 0, SIZE_MAX), TW_EUNSUPPORTED);

    if (g_fail) {
        std::printf("%d failures\n", g_fail);
        return 1;
    }
    std::printf("HARNESS_OK\n");
    return 0;
}
