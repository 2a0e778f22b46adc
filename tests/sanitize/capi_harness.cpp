// capi_harness.cpp -- drives every entry point of the C ABI through its
// argument validation and size arithmetic, for a host-only build of the
// library under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// It must run where no GPU is visible: calls that pass validation then fail
// at their first launch (no device), so the made-up device addresses below
// are never dereferenced.  It refuses to run if a device is present.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#include "samu_scan.h"

static int g_checks = 0;

static void expect(bool ok, const char* what, int line) {
    ++g_checks;
    if (!ok) {
        std::fprintf(stderr, "harness check failed at line %d: %s (last error: %s)\n", line, what,
                     scan_last_error());
        std::exit(2);
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
static float* F(uintptr_t a) { return reinterpret_cast<float*>(a); }

int main() {
    int n = -1;
    if (hipGetDeviceCount(&n) == hipSuccess && n > 0) {
        std::fprintf(stderr, "a GPU is visible: this harness runs only without one\n");
        return 3;
    }
    // ---- size queries over ordinary and extreme shapes: no UB, no overflow
    const int Bs[] = {0, 1, 3, 65535, 65536};
    const int Ls[] = {0, 1, 31, 32, 33, 1 << 20, 2147483647};
    const int Ds[] = {0, 2, 8, 12, 2048, 2560, 1 << 20};
    const int Ks[] = {8, 16, 32};
    const int Gs[] = {-1, 0, 1, 8, 16, 17, 1 << 30};
    size_t sink = 0;
    for (int B : Bs)
        for (int L : Ls)
            for (int D : Ds)
                for (int K : Ks) {
                    sink += samu_scan_saved_bytes(B, L, D, K) + rglru_scan_saved_bytes(B, L, D, K);
                    for (int G : Gs)
                        for (int bw = 0; bw < 2; ++bw)
                            sink += samu_scan_workspace_bytes(B, L, D, K, G, bw) +
                                    rglru_scan_workspace_bytes(B, L, D, K, G, bw) +
                                    scan_prefix_scratch_bytes(B, L, D, K, G, bw);
                }
    for (int v = -1; v < 3; ++v)
        for (int B : Bs)
            for (int L : Ls)
                for (int D : Ds)
                    sink += samu_scan_baseline_workspace_bytes(v, B, L, D) +
                            rglru_scan_baseline_workspace_bytes(v, B, L, D) +
                            rglru_gate_proj_bwd_workspace_bytes(B, L, D);
    for (int D : Ds) sink += samu_scan_decode_table_bytes(D);
    EXPECT(samu_scan_workspace_bytes(1, 0, 16, 32, 0, 0) == 0);
    EXPECT(samu_scan_saved_bytes(65536, 8, 16, 32) == 0);
    EXPECT(rglru_scan_saved_bytes(1, 2147483647, 2, 16) == 0);  // more than 65535 chunks

    // ---- every entry point, invalid arguments first, then arguments that
    // pass validation and fail at launch (no device)
    const uintptr_t X = 0x100000, Bd = 0x200000, W1 = 0x300000, W2 = 0x300100, A1 = 0x300200, A2 = 0x300210,
                    NU = 0x300300, TH = 0x300400, Y = 0x400000, SV = 0x500000, WS = 0x600000;
    const int B = 1, L = 64, D = 16, K = 32;
    const size_t wsf = samu_scan_workspace_bytes(B, L, D, K, 0, 0), wsb = samu_scan_workspace_bytes(B, L, D, K, 0, 1);
    EXPECT(samu_scan_fwd(B, L, 12, K, 0, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr, P(Y), 0,
                         nullptr, P(SV), P(WS), wsf, nullptr) == SCAN_ERR_SHAPE);
    EXPECT(samu_scan_fwd(B, L, D, K, 0, nullptr, P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr, P(Y), 0,
                         nullptr, P(SV), P(WS), wsf, nullptr) == SCAN_ERR_NULL);
    EXPECT(samu_scan_fwd(B, L, D, K, 0, P(X + 4), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr, P(Y),
                         0, nullptr, P(SV), P(WS), wsf, nullptr) == SCAN_ERR_ALIGN);
    EXPECT(samu_scan_fwd(B, L, D, K, 0, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr, P(Y), 0,
                         nullptr, P(SV), P(WS), wsf - 1, nullptr) == SCAN_ERR_WORKSPACE);
    EXPECT(samu_scan_fwd(B, L, D, K, 0, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr, P(X), 0,
                         nullptr, P(SV), P(WS), wsf, nullptr) == SCAN_ERR_ALIAS);
    for (int G : {0, 1, 2, 16, 17, 1000})
        for (int dt : {0, 1})
            EXPECT(samu_scan_fwd(B, L, D, K, G, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr,
                                 P(Y), dt, nullptr, P(SV), P(WS), samu_scan_workspace_bytes(B, L, D, K, G, 0),
                                 nullptr) == SCAN_ERR_DEVICE);
    EXPECT(samu_scan_fwd_noalloc(16, 131072, 2048, 32, 0, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH),
                                 nullptr, P(Y), 0, nullptr, P(SV), nullptr) == SCAN_ERR_WORKSPACE);
    for (int G : {0, 1, 17})
        EXPECT(samu_scan_bwd(B, L, D, K, G, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), P(SV),
                             P(0x700000), nullptr, P(0x800000), P(0x900000), 0, nullptr, F(0xa00000), F(0xa10000),
                             F(0xa20000), F(0xa20010), F(0xa30000), F(0xa40000), P(WS),
                             samu_scan_workspace_bytes(B, L, D, K, G, 1), nullptr) == SCAN_ERR_DEVICE);
    EXPECT(samu_scan_bwd(B, L, D, K, 0, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), P(SV), P(0x700000),
                         nullptr, P(0x800000), P(0x900000), 0, nullptr, F(0xa00000), F(0xa10000), F(0xa20000),
                         F(0xa20010), F(0xa30000), F(0xa40000), P(WS), wsb - 16, nullptr) == SCAN_ERR_WORKSPACE);
    EXPECT(samu_scan_decode(2, D, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr, nullptr,
                            F(0x700000), P(0x800000), 0, nullptr) == SCAN_ERR_DEVICE);
    EXPECT(samu_scan_decode_prepare(D, F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), P(0x800000), nullptr) ==
           SCAN_ERR_DEVICE);
    const size_t rwf = rglru_scan_workspace_bytes(4, 100, 10, 16, 0, 0), rwb = rglru_scan_workspace_bytes(4, 100, 10, 16, 0, 1);
    EXPECT(rglru_scan_fwd(4, 100, 10, 16, 0, P(X), P(Bd), P(W1), F(0x380000), nullptr, nullptr, P(Y), 0, nullptr,
                          P(SV), P(WS), rwf, nullptr) == SCAN_ERR_DEVICE);
    EXPECT(rglru_scan_bwd(4, 100, 10, 16, 0, P(X), P(Bd), P(W1), F(0x380000), nullptr, P(SV), P(0x700000), nullptr,
                          P(0x800000), P(0x900000), P(0x980000), 0, F(0xa00000), nullptr, P(WS), rwb, nullptr) ==
           SCAN_ERR_DEVICE);
    EXPECT(rglru_scan_fwd(4, 100, 9, 16, 0, P(X), P(Bd), P(W1), F(0x380000), nullptr, nullptr, P(Y), 0, nullptr,
                          P(SV), P(WS), rwf, nullptr) == SCAN_ERR_SHAPE);
    for (int v : {0, 1}) {
        EXPECT(samu_scan_baseline_fwd(v, 2, 33, D, P(X), P(Bd), F(W1), F(W2), F(A1), F(A2), F(NU), F(TH), nullptr,
                                      P(Y), 0, nullptr, P(WS), samu_scan_baseline_workspace_bytes(v, 2, 33, D),
                                      nullptr) == SCAN_ERR_DEVICE);
        const size_t rb = rglru_scan_baseline_workspace_bytes(v, 2, 33, 10);
        EXPECT(rglru_scan_baseline_fwd(v, 2, 33, 10, P(X), P(Bd), P(W1), F(0x380000), nullptr, nullptr, P(Y), 0,
                                       nullptr, rb ? P(WS) : nullptr, rb, nullptr) == SCAN_ERR_DEVICE);
    }
    EXPECT(rglru_gate_proj_fwd(1, 8, 256, P(X), P(0x310000), F(0x320000), P(0x330000), F(0x340000), P(0x500000),
                               P(0x580000), nullptr) == SCAN_ERR_DEVICE);
    EXPECT(rglru_gate_proj_bwd(1, 8, 256, P(X), P(0x310000), P(0x330000), P(0x400000), P(0x480000), 0,
                               P(0x500000), P(0x500000), F(0x700000), F(0x710000), F(0x720000), F(0x730000),
                               P(0x800000), rglru_gate_proj_bwd_workspace_bytes(1, 8, 256), nullptr) ==
           SCAN_ERR_DEVICE);
    // profiler bookkeeping with nothing recorded
    scan_profile_enable(1);
    scan_profile_enable(0);
    for (int k = -1; k <= scan_profile_kernel_count(); ++k) sink += (size_t)scan_profile_kernel_name(k)[0];
    double ms[64];
    int cnt[64];
    EXPECT(scan_profile_kernel_count() <= 64);
    EXPECT(scan_profile_collect(ms, cnt) == SCAN_OK);
    std::printf("capi harness: %d checks passed (%zu)\n", g_checks, sink & 1);
    return 0;
}
