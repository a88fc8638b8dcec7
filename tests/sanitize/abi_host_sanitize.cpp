// Host-side paths of the C ABI (include/ep.h) that run without a GPU: the
// workspace sizing of ep_workspace_bytes / ep_ec_workspace_bytes over a wide
// grid of sizes, up to T*K and E*C near 2^31, and the argument checks of all
// six entry points, which must return their status before anything is
// enqueued.  Built with the host pass under AddressSanitizer and
// UndefinedBehaviorSanitizer, so that an overflow in the size arithmetic or
// an access outside a host object is reported.  Exit status 0 = clean.
// Test infrastructure: built and run by tests/test_abi_sanitize.py.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "ep.h"

static int failures = 0;

static void expect(bool ok, const char *what, long long a, long long b)
{
    if (!ok) {
        fprintf(stderr, "%s (%lld, %lld)\n", what, a, b);
        ++failures;
    }
}

int main()
{
    const int Ks[] = {1, 2, 7, 8, 16, 40, 64, 257, 1024};
    const int Es[] = {1, 2, 8, 37, 256, 384, 1000, 4096};
    const long long Ts[] = {0, 1, 63, 64, 65, 128, 4095, 4096, 16384, 300000, 1 << 20};
    for (int K : Ks)
        for (int E : Es)
            for (long long T : Ts) {
                const int R = E % 8 == 0 ? 8 : 1;
                const size_t b = ep_workspace_bytes((int)T, K, E, R);
                expect(b > 0 && b % 256 == 0, "workspace size positive and 256-aligned", T, K);
                expect(b >= (size_t)T * K * 4, "workspace holds one int per entry", T, K);
            }
    // the largest token counts a top-k allows (T*K just below 2^31)
    for (int K : Ks) {
        const long long T = 2147483647LL / K;
        const size_t b = ep_workspace_bytes((int)T, K, 4096, 1024);
        expect(b >= (size_t)T * K * 4, "largest plan holds every entry", T, K);
        if (T + 1 <= 2147483647LL)
            expect(ep_workspace_bytes((int)(T + 1), K, 4096, 1024) == 0, "T*K beyond 2^31 is refused",
                   T + 1, K);
    }
    expect(ep_workspace_bytes(-1, 8, 256, 1) == 0, "negative T", -1, 0);
    expect(ep_workspace_bytes(10, 0, 256, 1) == 0, "K = 0", 0, 0);
    expect(ep_workspace_bytes(10, 8, 4097, 1) == 0, "E beyond 4096", 4097, 0);
    expect(ep_workspace_bytes(10, 8, 256, 3) == 0, "E % R != 0", 256, 3);
    expect(ep_workspace_bytes(10, 1025, 256, 1) > 0, "K beyond 1024 is accepted", 1025, 0);
    expect(ep_workspace_bytes(5, 1 << 29, 256, 1) == 0, "T*K beyond 2^31", 5, 1 << 29);

    const long long Cs[] = {1, 3, 256, 4096, 1 << 20};
    for (long long C : Cs)
        for (int E : Es)
            for (long long T : Ts) {
                if ((long long)E * C > 2147483647LL) {
                    expect(ep_ec_workspace_bytes((int)T, E, (int)C) == 0, "E*C beyond 2^31", E, C);
                    continue;
                }
                const size_t b = ep_ec_workspace_bytes((int)T, E, (int)C);
                expect(b >= (size_t)E * C * 4 + (size_t)(T + 1) * 8, "EC workspace", E, C);
            }

    // argument checks: every one returns before anything touches a device
    alignas(256) static char ws[1 << 16];
    int32_t i4[64] = {0};
    uint16_t h2[64] = {0};
    float f4[64] = {0};
    uint8_t u1[64] = {0};
    const ep_status_t inval = EP_ERR_INVALID_ARG, unsup = EP_ERR_UNSUPPORTED;
    expect(ep_get_dispatch_layout(nullptr, 4, 2, 8, 1, i4, i4, i4, u1, i4, ws, sizeof ws,
                                  nullptr) == inval, "layout: null topk_idx", 0, 0);
    expect(ep_get_dispatch_layout(i4, 4, 2, 8, 1, i4, i4, i4, u1, i4, nullptr, sizeof ws,
                                  nullptr) == EP_ERR_WORKSPACE, "layout: null workspace", 0, 0);
    expect(ep_get_dispatch_layout(i4, 4, 2, 8, 1, i4, i4, i4, u1, i4, ws + 8, sizeof ws - 8,
                                  nullptr) == EP_ERR_WORKSPACE, "layout: misaligned workspace", 0, 0);
    expect(ep_get_dispatch_layout(i4, 4, 2, 5000, 1, i4, i4, i4, u1, i4, ws, sizeof ws,
                                  nullptr) == unsup, "layout: E beyond 4096", 0, 0);
    expect(ep_dispatch(h2, 4, 12, i4, 2, 8, i4, EP_LAYOUT_CONTIGUOUS, 8, EP_QUANT_BF16, h2, nullptr,
                       i4, i4, i4, ws, sizeof ws, nullptr) == inval, "dispatch: H % 8", 12, 0);
    expect(ep_dispatch(h2, 4, 64, i4, 2, 8, i4, EP_LAYOUT_CONTIGUOUS, 8, EP_QUANT_FP8_E4M3_G128,
                       h2, f4, i4, i4, i4, ws, sizeof ws, nullptr) == inval, "dispatch: fp8 H % 128", 64, 0);
    expect(ep_dispatch(h2, 4, 1 << 25, i4, 2, 8, i4, EP_LAYOUT_CONTIGUOUS, 8, EP_QUANT_BF16, h2,
                       nullptr, i4, i4, i4, ws, sizeof ws, nullptr) == unsup, "dispatch: H beyond 2^24", 0, 0);
    expect(ep_dispatch(h2, 4, 64, i4, 2, 8, i4, EP_LAYOUT_PADDED, 1 << 30, EP_QUANT_BF16, h2,
                       nullptr, i4, i4, i4, ws, sizeof ws, nullptr) == inval, "dispatch: E*cap beyond 2^31", 0, 0);
    expect(ep_dispatch(h2, 4, 64, i4, 2, 8, i4, (ep_recv_layout_t)7, 8, EP_QUANT_BF16, h2, nullptr,
                       i4, i4, i4, ws, sizeof ws, nullptr) == inval, "dispatch: layout enum", 7, 0);
    expect(ep_dispatch(h2, 4, 64, i4, 2, 8, i4, EP_LAYOUT_CONTIGUOUS, 8, (ep_quant_t)9, h2, nullptr,
                       i4, i4, i4, ws, sizeof ws, nullptr) == inval, "dispatch: quant enum", 9, 0);
    // the one-launch low-latency dispatch: limits and argument checks
    expect(ep_low_latency_dispatch(h2, 4097, 64, i4, 1, 8, 4, EP_QUANT_BF16, h2, nullptr, i4, i4,
                                   i4, i4, i4, nullptr) == unsup, "ll: T*K beyond 4096", 4097, 1);
    expect(ep_low_latency_dispatch(h2, 1, 64, i4, 65, 8, 4, EP_QUANT_BF16, h2, nullptr, i4, i4, i4,
                                   i4, i4, nullptr) == unsup, "ll: K beyond 64", 1, 65);
    expect(ep_low_latency_dispatch(h2, 4, 8320, i4, 2, 8, 4, EP_QUANT_INT8_TOKEN, u1, f4, i4, i4,
                                   i4, i4, i4, nullptr) == unsup, "ll: per-token row of 520 pairs",
           8320, 0);
    expect(ep_low_latency_dispatch(h2, 4, 4104, i4, 2, 8, 4, EP_QUANT_FP8_E4M3_TOKEN, u1, f4, i4,
                                   i4, i4, i4, i4, nullptr) == unsup,
           "ll: per-token row of 513 pieces", 4104, 0);
    expect(ep_low_latency_dispatch(h2, 4, 64, i4, 2, 8, -1, EP_QUANT_BF16, h2, nullptr, i4, i4, i4,
                                   i4, i4, nullptr) == inval, "ll: cap < 0", -1, 0);
    expect(ep_low_latency_dispatch(h2, 4, 64, i4, 2, 4096, 1 << 20, EP_QUANT_BF16, h2, nullptr, i4,
                                   i4, i4, i4, i4, nullptr) == inval, "ll: E*cap beyond 2^31", 0, 0);
    expect(ep_low_latency_dispatch(h2, 4, 64, i4, 2, 8, 4, 9, h2, nullptr, i4, i4, i4, i4, i4,
                                   nullptr) == inval, "ll: quant code", 9, 0);
    expect(ep_low_latency_dispatch(h2, 4, 64, i4, 2, 8, 4, EP_QUANT_FP8_E4M3_G128, u1, f4, i4, i4,
                                   i4, i4, i4, nullptr) == inval, "ll: fp8 H % 128", 64, 0);
    expect(ep_low_latency_dispatch(h2, 4, 64, i4, 2, 8, 4, EP_QUANT_BF16, h2, nullptr, i4, i4,
                                   nullptr, i4, i4, nullptr) == inval, "ll: null recv_count", 0, 0);
    expect(ep_low_latency_dispatch(h2, 4, 64, i4, 2, 5000, 4, EP_QUANT_BF16, h2, nullptr, i4, i4,
                                   i4, i4, i4, nullptr) == unsup, "ll: E beyond 4096", 5000, 0);
    expect(ep_combine(h2, 8, 64, i4, f4, -1, 2, h2, nullptr) == inval, "combine: T < 0", 0, 0);
    expect(ep_combine(h2, 8, 64, nullptr, f4, 4, 2, h2, nullptr) == inval, "combine: null slot", 0, 0);
    expect(ep_combine(h2, 8, 64, i4, f4, 1 << 30, 8, h2, nullptr) == inval, "combine: T*K beyond 2^31", 0, 0);
    expect(ep_dispatch_expert_choice(h2, 4, 64, i4, 1 << 16, 1 << 16, h2, i4, i4, i4, ws, sizeof ws,
                                     nullptr) == inval, "ec dispatch: E*C beyond 2^31", 0, 0);
    expect(ep_dispatch_expert_choice(h2, 4, 64, nullptr, 2, 2, h2, i4, i4, i4, ws, sizeof ws,
                                     nullptr) == inval, "ec dispatch: null indices", 0, 0);
    expect(ep_combine_expert_choice(h2, f4, 2, 2, 12, i4, i4, 4, h2, nullptr) == inval,
           "ec combine: H % 8", 12, 0);
    for (int s = 0; s <= 5; ++s)
        expect(ep_status_string((ep_status_t)s)[0] != 0, "status string", s, 0);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi host sanitize run clean\n");
    return 0;
}
