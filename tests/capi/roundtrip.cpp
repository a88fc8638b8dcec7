// A plain C++ host program that uses libep only through include/ep.h:
// hipMalloc'd buffers, the six entry points on the null stream, hipMemcpy
// back.  It checks properties that hold at any size, without the oracle:
//   token choice ("DeepEP-Ascend" README, API Overview): counts sum to the
//   valid (t,k); offsets are their exclusive prefix; slots are a bijection
//   onto [0, N) with each expert's rows in ascending (t,k); every received
//   row equals its source row; with unit weights the combine gives
//   bf16(m_t * x_t) exactly (m_t = the token's kept slots; every partial sum
//   is exact in fp32), and +0 for a token with none;
//   expert choice ("[Feature Request] Support Expert-Choice Routing via
//   Native Expert-Centric API", Solution 1): the inverse map lists each
//   token's entries in ascending order, received rows equal their tokens'
//   rows, and the unit-weight combine gives bf16(picks_t * x_t);
//   the one-launch low-latency dispatch: expert e's rows in ascending (t,k)
//   from e*cap, capacity overflow dropped and counted, recv_count.
// Exit status 0 = every check passed.  Built by tests/capi/build.py.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "ep.h"

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                \
            return 2;                                                                 \
        }                                                                             \
    } while (0)
#define EP_OK_(call)                                                                  \
    do {                                                                              \
        ep_status_t s_ = (call);                                                      \
        if (s_ != EP_OK) {                                                            \
            fprintf(stderr, "%s: %s\n", #call, ep_status_string(s_));                 \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

static uint64_t st = 0x2545F4914F6CDD1Dull;
static uint32_t rnd() { st = st * 6364136223846793005ull + 1442695040888963407ull; return (uint32_t)(st >> 33); }

static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// Nearest bf16 to an fp32 value that is a product m*x with m <= 2^16 (so
// finite and, when not zero, normal), ties to even, from its decomposition.
static uint16_t bf16_nearest(float v)
{
    if (v == 0.0f)
        return 0;                               // sums start from +0
    int e;
    const double m = frexp(fabs((double)v), &e);    // v = m * 2^e, m in [0.5, 1)
    const double q = nearbyint(ldexp(m, 8));         // 8 significant bits, ties to even
    const float r = (float)ldexp(q, e - 8);
    uint32_t u;
    memcpy(&u, &r, 4);
    return (uint16_t)((u >> 16) | (v < 0 ? 0x8000u : 0u));
}

static int failures = 0;
static void expect(bool ok, const char *what, long a)
{
    if (!ok && failures++ < 20)
        fprintf(stderr, "check failed: %s (%ld)\n", what, a);
}

static int token_choice()
{
    const int T = 3000, H = 1024, E = 64, K = 6;
    const int64_t TK = (int64_t)T * K;
    std::vector<int32_t> idx(TK);
    for (auto &v : idx) {
        const uint32_t u = rnd() % 100;
        v = u < 8 ? -1 : (int32_t)(u < 20 ? rnd() % 4 : rnd() % E);   // padding; hot experts
    }
    std::vector<uint16_t> x((size_t)T * H);
    for (auto &v : x)
        v = (uint16_t)(((rnd() & 1u) << 15) | ((uint32_t)(110 + rnd() % 30) << 7) | (rnd() & 0x7Fu));
    const int rows = (int)TK;
    int32_t *d_idx, *d_counts, *d_off, *d_ninv, *d_slot, *d_src, *d_nd;
    uint16_t *d_x, *d_recv, *d_out;
    void *d_ws;
    const size_t wsb = ep_workspace_bytes(T, K, E, 1);
    HIP_OK(hipMalloc(&d_idx, TK * 4));
    HIP_OK(hipMalloc(&d_counts, E * 4));
    HIP_OK(hipMalloc(&d_off, (E + 1) * 4));
    HIP_OK(hipMalloc(&d_ninv, 4));
    HIP_OK(hipMalloc(&d_slot, TK * 4));
    HIP_OK(hipMalloc(&d_src, (size_t)rows * 4));
    HIP_OK(hipMalloc(&d_nd, 4));
    HIP_OK(hipMalloc(&d_x, (size_t)T * H * 2));
    HIP_OK(hipMalloc(&d_recv, (size_t)rows * H * 2));
    HIP_OK(hipMalloc(&d_out, (size_t)T * H * 2));
    HIP_OK(hipMalloc(&d_ws, wsb));
    HIP_OK(hipMemcpy(d_idx, idx.data(), TK * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x.data(), (size_t)T * H * 2, hipMemcpyHostToDevice));

    EP_OK_(ep_get_dispatch_layout(d_idx, T, K, E, 1, d_counts, d_off, nullptr, nullptr, d_ninv,
                                  d_ws, wsb, nullptr));
    EP_OK_(ep_dispatch(d_x, T, H, d_idx, K, E, d_off, EP_LAYOUT_CONTIGUOUS, rows, EP_QUANT_BF16,
                       d_recv, nullptr, d_slot, d_src, d_nd, d_ws, wsb, nullptr));
    EP_OK_(ep_combine(d_recv, rows, H, d_slot, nullptr, T, K, d_out, nullptr));
    HIP_OK(hipDeviceSynchronize());

    std::vector<int32_t> counts(E), off(E + 1), slot(TK), src(rows);
    std::vector<uint16_t> recv((size_t)rows * H), out((size_t)T * H);
    int32_t ninv, nd;
    HIP_OK(hipMemcpy(counts.data(), d_counts, E * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(off.data(), d_off, (E + 1) * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(slot.data(), d_slot, TK * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(src.data(), d_src, (size_t)rows * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv.data(), d_recv, (size_t)rows * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out.data(), d_out, (size_t)T * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&ninv, d_ninv, 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&nd, d_nd, 4, hipMemcpyDeviceToHost));

    int64_t valid = 0;
    for (int32_t v : idx)
        valid += v >= 0;
    int64_t sum = 0;
    for (int e = 0; e < E; ++e) {
        expect(off[e] == sum, "offsets are the exclusive prefix of counts", e);
        sum += counts[e];
    }
    expect(sum == valid && off[E] == valid, "counts sum to the valid slots", (long)sum);
    expect(ninv == 0 && nd == 0, "no invalid entry, nothing dropped", ninv);
    std::vector<char> hit(rows, 0);
    std::vector<int> last(E, -1), m(T, 0);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            const int e = idx[(int64_t)t * K + k], s = slot[(int64_t)t * K + k];
            if (e < 0) {
                expect(s == -1, "padding gets no slot", t);
                continue;
            }
            expect(s >= off[e] && s < off[e + 1], "slot inside its expert's block", s);
            if (s < 0 || s >= rows)
                continue;
            expect(!hit[s], "no slot taken twice", s);
            hit[s] = 1;
            expect(s > last[e], "ascending (t,k) inside an expert", s);
            last[e] = s;
            expect(src[s] == t, "recv_src is the source token", s);
            expect(memcmp(&recv[(size_t)s * H], &x[(size_t)t * H], (size_t)H * 2) == 0,
                   "received row equals its source row", s);
            ++m[t];
        }
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            const float p = (float)m[t] * bf16_value(x[(size_t)t * H + h]);
            expect(out[(size_t)t * H + h] == bf16_nearest(p), "unit-weight combine = bf16(m_t x_t)", t);
        }
    hipFree(d_idx); hipFree(d_counts); hipFree(d_off); hipFree(d_ninv); hipFree(d_slot);
    hipFree(d_src); hipFree(d_nd); hipFree(d_x); hipFree(d_recv); hipFree(d_out); hipFree(d_ws);
    return 0;
}

static int expert_choice()
{
    const int T = 1000, H = 512, E = 16, C = 64;
    const int n = E * C;
    std::vector<int32_t> ti(n);
    for (auto &v : ti)
        v = rnd() % 10 == 0 ? -1 : (int32_t)(rnd() % 5 == 0 ? rnd() % 8 : rnd() % T);  // hot tokens
    std::vector<uint16_t> x((size_t)T * H);
    for (auto &v : x)
        v = (uint16_t)(((rnd() & 1u) << 15) | ((uint32_t)(110 + rnd() % 30) << 7) | (rnd() & 0x7Fu));
    std::vector<float> w(n, 1.0f);
    int32_t *d_ti, *d_off, *d_ent, *d_ninv;
    uint16_t *d_x, *d_recv, *d_out;
    float *d_w;
    void *d_ws;
    const size_t wsb = ep_ec_workspace_bytes(T, E, C);
    HIP_OK(hipMalloc(&d_ti, n * 4));
    HIP_OK(hipMalloc(&d_off, (T + 1) * 4));
    HIP_OK(hipMalloc(&d_ent, n * 4));
    HIP_OK(hipMalloc(&d_ninv, 4));
    HIP_OK(hipMalloc(&d_x, (size_t)T * H * 2));
    HIP_OK(hipMalloc(&d_recv, (size_t)n * H * 2));
    HIP_OK(hipMalloc(&d_out, (size_t)T * H * 2));
    HIP_OK(hipMalloc(&d_w, n * 4));
    HIP_OK(hipMalloc(&d_ws, wsb));
    HIP_OK(hipMemcpy(d_ti, ti.data(), n * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x.data(), (size_t)T * H * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_w, w.data(), n * 4, hipMemcpyHostToDevice));

    EP_OK_(ep_dispatch_expert_choice(d_x, T, H, d_ti, E, C, d_recv, d_off, d_ent, d_ninv, d_ws, wsb,
                                     nullptr));
    EP_OK_(ep_combine_expert_choice(d_recv, d_w, E, C, H, d_off, d_ent, T, d_out, nullptr));
    HIP_OK(hipDeviceSynchronize());

    std::vector<int32_t> off(T + 1), ent(n);
    std::vector<uint16_t> recv((size_t)n * H), out((size_t)T * H);
    HIP_OK(hipMemcpy(off.data(), d_off, (T + 1) * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(ent.data(), d_ent, n * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv.data(), d_recv, (size_t)n * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out.data(), d_out, (size_t)T * H * 2, hipMemcpyDeviceToHost));

    std::vector<int> picks(T, 0);
    int valid = 0;
    for (int j = 0; j < n; ++j)
        if (ti[j] >= 0) {
            ++picks[ti[j]];
            ++valid;
            expect(memcmp(&recv[(size_t)j * H], &x[(size_t)ti[j] * H], (size_t)H * 2) == 0,
                   "received row equals its token's row", j);
        }
    expect(off[0] == 0 && off[T] == valid, "the map holds every valid entry", off[T]);
    for (int t = 0; t < T; ++t) {
        expect(off[t + 1] - off[t] == picks[t], "a token's entry count", t);
        for (int a = off[t]; a < off[t + 1] && a >= 0 && a < n; ++a) {
            const bool in_range = ent[a] >= 0 && ent[a] < n;
            expect(in_range && ti[ent[a]] == t, "an entry of the token", a);
            expect(a == off[t] || ent[a] > ent[a - 1], "entries ascending", a);
        }
        for (int h = 0; h < H; ++h) {
            const float p = (float)picks[t] * bf16_value(x[(size_t)t * H + h]);
            expect(out[(size_t)t * H + h] == bf16_nearest(p), "unit-weight combine = bf16(picks_t x_t)", t);
        }
    }
    hipFree(d_ti); hipFree(d_off); hipFree(d_ent); hipFree(d_ninv); hipFree(d_x);
    hipFree(d_recv); hipFree(d_out); hipFree(d_w); hipFree(d_ws);
    return 0;
}

// The one-launch low-latency dispatch into [E, cap] rows with overflow:
// expert e's rows are e*cap + 0, 1, ... in ascending (t,k), entries beyond
// cap get -1; recv_count, num_dropped and num_invalid follow from the
// per-expert counts; rows equal their sources and the unit-weight combine
// over the padded rows gives bf16(m_t * x_t).
static int low_latency()
{
    const int T = 128, H = 512, E = 32, K = 6, cap = 12;
    const int TK = T * K, rows = E * cap;
    std::vector<int32_t> idx(TK);
    for (auto &v : idx) {
        const uint32_t u = rnd() % 100;
        v = u < 10 ? -1 : (int32_t)(u < 30 ? rnd() % 3 : rnd() % E);   // padding; hot experts
    }
    std::vector<uint16_t> x((size_t)T * H);
    for (auto &v : x)
        v = (uint16_t)(((rnd() & 1u) << 15) | ((uint32_t)(110 + rnd() % 30) << 7) | (rnd() & 0x7Fu));
    int32_t *d_idx, *d_slot, *d_src, *d_cnt, *d_nd, *d_ninv;
    uint16_t *d_x, *d_recv, *d_out;
    HIP_OK(hipMalloc(&d_idx, TK * 4));
    HIP_OK(hipMalloc(&d_slot, TK * 4));
    HIP_OK(hipMalloc(&d_src, rows * 4));
    HIP_OK(hipMalloc(&d_cnt, E * 4));
    HIP_OK(hipMalloc(&d_nd, 4));
    HIP_OK(hipMalloc(&d_ninv, 4));
    HIP_OK(hipMalloc(&d_x, (size_t)T * H * 2));
    HIP_OK(hipMalloc(&d_recv, (size_t)rows * H * 2));
    HIP_OK(hipMalloc(&d_out, (size_t)T * H * 2));
    HIP_OK(hipMemcpy(d_idx, idx.data(), TK * 4, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(d_x, x.data(), (size_t)T * H * 2, hipMemcpyHostToDevice));

    EP_OK_(ep_low_latency_dispatch(d_x, T, H, d_idx, K, E, cap, EP_QUANT_BF16, d_recv, nullptr,
                                   d_slot, d_src, d_cnt, d_nd, d_ninv, nullptr));
    EP_OK_(ep_combine(d_recv, rows, H, d_slot, nullptr, T, K, d_out, nullptr));
    HIP_OK(hipDeviceSynchronize());

    std::vector<int32_t> slot(TK), src(rows), cnt(E);
    std::vector<uint16_t> recv((size_t)rows * H), out((size_t)T * H);
    int32_t nd, ninv;
    HIP_OK(hipMemcpy(slot.data(), d_slot, TK * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(src.data(), d_src, rows * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(cnt.data(), d_cnt, E * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(recv.data(), d_recv, (size_t)rows * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out.data(), d_out, (size_t)T * H * 2, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&nd, d_nd, 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(&ninv, d_ninv, 4, hipMemcpyDeviceToHost));

    std::vector<int> next(E, 0), m(T, 0);
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            const int e = idx[t * K + k], s = slot[t * K + k];
            if (e < 0) {
                expect(s == -1, "ll: padding gets no slot", t);
                continue;
            }
            const int r = next[e]++;
            expect(s == (r < cap ? e * cap + r : -1), "ll: expert rows in ascending (t,k)", s);
            if (s < 0)
                continue;
            expect(src[s] == t, "ll: recv_src is the source token", s);
            expect(memcmp(&recv[(size_t)s * H], &x[(size_t)t * H], (size_t)H * 2) == 0,
                   "ll: received row equals its source row", s);
            ++m[t];
        }
    int dropped = 0;
    for (int e = 0; e < E; ++e) {
        expect(cnt[e] == (next[e] < cap ? next[e] : cap), "ll: recv_count = min(count, cap)", e);
        dropped += next[e] > cap ? next[e] - cap : 0;
    }
    expect(dropped > 0 && nd == dropped, "ll: num_dropped", nd);
    expect(ninv == 0, "ll: no invalid entry", ninv);
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h) {
            const float p = (float)m[t] * bf16_value(x[(size_t)t * H + h]);
            expect(out[(size_t)t * H + h] == bf16_nearest(p), "ll: unit-weight combine", t);
        }
    hipFree(d_idx); hipFree(d_slot); hipFree(d_src); hipFree(d_cnt); hipFree(d_nd);
    hipFree(d_ninv); hipFree(d_x); hipFree(d_recv); hipFree(d_out);
    return 0;
}

int main()
{
    int dev_count = 0;
    HIP_OK(hipGetDeviceCount(&dev_count));
    if (dev_count < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    if (token_choice() || low_latency() || expert_choice())
        return 2;
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("capi roundtrip ok\n");
    return 0;
}
