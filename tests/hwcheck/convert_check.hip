// convert_check.hip -- test-only library: exhaustive GPU checks of the
// dispatch kernel's element arithmetic (the helpers in ep_common.h) against
// software definitions written here.
//
//   * e4m3x4 / e5m2x4 (gfx950 conversion instructions) against software
//     round-to-nearest-even encoders of the OCP E4M3 and E5M2 formats, for
//     every finite fp32 input: unbounded below the saturation midpoint (464,
//     61440) and bounded with med3 (as the MX modes do) everywhere; each of
//     the four byte positions.
//   * e2m1x8_scaled against x * 2^-E then a software E2M1 encoder, for every
//     finite bf16 x and every E in [-127, 125] with |x| * 2^-E < 8 (every
//     MX block value), each of the eight nibble positions; and with E = 0
//     for every finite fp32 input.
//   * div_by_scale (with the IEEE fallback below kFastDivMinScale, as the
//     kernel uses it) against the correctly rounded x / s, for every pair of
//     finite bf16 amax > 0 and bf16 |x| <= amax with s = amax/448 and
//     s = amax/127: equal E4M3 / int8 codes, and equal fp32 quotients when
//     |x / s| >= 2^-11.
//
// Host entry: convert_check(counts) fills counts[kNumCounters] (mismatches,
// then the number of cases each check saw) and returns 0, or a HIP error.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_common.h"

namespace {

using ep::div_by_scale;
using ep::e2m1x8_scaled;
using ep::e4m3x4;
using ep::e5m2x4;
using ep::f32_to_int8_rne;
using ep::kFastDivMinScale;

// ------------------------------------------------- software encoders
// fp32 -> E4M3 (bias 7, 3 mantissa bits, largest finite 448), nearest even.
// Below 2^-6 the code is the subnormal count round(|v| * 2^9); from 2^-6 up
// the pattern is rounded to 3 mantissa bits in place (a carry moves into the
// exponent) and rebiased.  |v| >= 464 saturates to 448.
__device__ uint32_t sw_e4m3(float v)
{
    const uint32_t u = __float_as_uint(v), sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E80000u)
        code = 0x7Eu;
    else if (a < 0x3C800000u)
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    else {
        const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
        code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
    }
    return sign | code;
}

// fp32 -> E5M2 (bias 15, 2 mantissa bits, largest finite 57344), nearest
// even, saturating at and above 61440.
__device__ uint32_t sw_e5m2(float v)
{
    const uint32_t u = __float_as_uint(v), sign = (u >> 24) & 0x80u, a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x47700000u)
        code = 0x7Bu;
    else if (a < 0x38800000u)
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 65536.0f);
    else {
        const uint32_t r = a + 0xFFFFFu + ((a >> 21) & 1u);
        code = (((r >> 23) - 112u) << 2) | ((r >> 21) & 3u);
    }
    return sign | code;
}

// fp32 -> E2M1 nibble (0, .5, 1, 1.5, 2, 3, 4, 6 = codes 0..7, bit 3 the
// sign), nearest even, saturating at 6.
__device__ uint32_t sw_e2m1(float v)
{
    const uint32_t u = __float_as_uint(v), sign = (u >> 28) & 0x8u, a = u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x40C00000u)
        code = 7u;
    else if (a < 0x3F800000u)
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 2.0f);
    else {
        const uint32_t r = a + 0x1FFFFFu + ((a >> 22) & 1u);
        code = (((r >> 23) - 126u) << 1) | ((r >> 22) & 1u);
    }
    return sign | code;
}

// ------------------------------------------------- counters
enum {
    kE4m3Raw, kE4m3Med3, kE5m2Raw, kE5m2Med3, kE2m1Fp32, kE2m1Mx,
    kDiv448Code, kDiv127Code, kDiv448F32, kDiv127F32, kDiv448HwCode,
    kNumChecks
};
constexpr int kNumCounters = 2 * kNumChecks;    // mismatches, then cases

__device__ unsigned long long g_counts[kNumCounters];

struct Tally {
    unsigned long long c[kNumCounters] = {};
    __device__ void note(int check, bool bad)
    {
        c[check] += bad ? 1u : 0u;
        c[kNumChecks + check] += 1u;
    }
    __device__ void flush()
    {
        for (int k = 0; k < kNumCounters; ++k)
            if (c[k])
                atomicAdd(&g_counts[k], c[k]);
    }
};

// byte k of the word from e4m3x4/e5m2x4 with v at position k, fixed values
// elsewhere
template <bool E5M2>
__device__ bool pos_ok(float v, uint32_t want)
{
    const float o[3] = {1.0f, -2.5f, 0.375f};
    bool ok = true;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float in[4];
        int m = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            in[p] = p == k ? v : o[m++ % 3];
        const uint32_t w = E5M2 ? e5m2x4(in[0], in[1], in[2], in[3])
                                : e4m3x4(in[0], in[1], in[2], in[3]);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t ref = p == k ? want : (E5M2 ? sw_e5m2(in[p]) : sw_e4m3(in[p]));
            ok = ok && ((w >> (8 * p)) & 0xFFu) == ref;
        }
    }
    return ok;
}

// every fp32 pattern, grid-stride
__global__ void __launch_bounds__(256) fp32_kernel()
{
    Tally t;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32);
         i += stride) {
        const uint32_t u = (uint32_t)i, a = u & 0x7FFFFFFFu;
        if (a >= 0x7F800000u)
            continue;                                      // inf, NaN
        const float v = __uint_as_float(u);
        if (a < 0x43E80000u)
            t.note(kE4m3Raw, !pos_ok<false>(v, sw_e4m3(v)));
        t.note(kE4m3Med3, !pos_ok<false>(__builtin_amdgcn_fmed3f(v, -448.0f, 448.0f), sw_e4m3(v)));
        if (a < 0x47700000u)
            t.note(kE5m2Raw, !pos_ok<true>(v, sw_e5m2(v)));
        t.note(kE5m2Med3,
               !pos_ok<true>(__builtin_amdgcn_fmed3f(v, -57344.0f, 57344.0f), sw_e5m2(v)));
        const float in[8] = {v, 0.5f, -1.5f, 3.0f, v, -0.0f, 6.0f, -0.25f};
        const uint32_t w = e2m1x8_scaled(in, 127u);
        bool ok = true;
#pragma unroll
        for (int p = 0; p < 8; ++p)
            ok = ok && ((w >> (4 * p)) & 0xFu) == sw_e2m1(in[p]);
        t.note(kE2m1Fp32, !ok);
    }
    t.flush();
}

// every finite bf16 x and E in [-127, 125] with |x| * 2^-E < 8
__global__ void __launch_bounds__(256) mx_e2m1_kernel()
{
    Tally t;
    const uint32_t total = 253u << 16;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += gridDim.x * blockDim.x) {
        const int E = (int)(i >> 16) - 127;
        const uint32_t xb = i & 0xFFFFu;
        if ((xb & 0x7F80u) == 0x7F80u)
            continue;
        const float x = __uint_as_float(xb << 16);
        const float m = __uint_as_float((uint32_t)(127 - E) << 23);    // 2^-E, normal
        if (!(fabsf(x) * m < 8.0f))
            continue;
        const int p = (int)(xb & 7u);                    // nibble position of x
        float in[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            in[q] = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q == p)
                in[q] = x;
        const uint32_t w = e2m1x8_scaled(in, (uint32_t)(E + 127));
        const uint32_t want = sw_e2m1(x * m);
        t.note(kE2m1Mx, w != (want << (4 * p)));
    }
    t.flush();
}

// every pair of bf16 amax > 0 (finite) and bf16 |x| <= amax
__global__ void __launch_bounds__(256) div_kernel()
{
    Tally t;
    const uint32_t total = 0x7F80u << 16;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += gridDim.x * blockDim.x) {
        const uint32_t ab = i >> 16, xb = i & 0xFFFFu;
        if (ab == 0u || (xb & 0x7FFFu) > ab)
            continue;
        const float amax = __uint_as_float(ab << 16), x = __uint_as_float(xb << 16);
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const float s = amax / (d ? 127.0f : 448.0f);
            const float ieee = x / s;
            const float q = s >= kFastDivMinScale ? div_by_scale(x, s, 1.0f / s) : x / s;
            if (d) {
                t.note(kDiv127Code, f32_to_int8_rne(q) != f32_to_int8_rne(ieee));
                if (fabsf(ieee) >= 0x1p-11f)
                    t.note(kDiv127F32, __float_as_uint(q) != __float_as_uint(ieee));
            } else {
                t.note(kDiv448Code, sw_e4m3(q) != sw_e4m3(ieee));
                t.note(kDiv448HwCode, (e4m3x4(q, 0.0f, 0.0f, 0.0f) & 0xFFu) != sw_e4m3(ieee));
                if (fabsf(ieee) >= 0x1p-11f)
                    t.note(kDiv448F32, __float_as_uint(q) != __float_as_uint(ieee));
            }
        }
    }
    t.flush();
}

}  // namespace

extern "C" int convert_check_num_counters() { return kNumCounters; }

extern "C" int convert_check(unsigned long long *counts)
{
    unsigned long long zero[kNumCounters] = {};
    hipError_t err = hipMemcpyToSymbol(HIP_SYMBOL(g_counts), zero, sizeof zero);
    if (err == hipSuccess) {
        hipLaunchKernelGGL(fp32_kernel, dim3(8192), dim3(256), 0, 0);
        hipLaunchKernelGGL(mx_e2m1_kernel, dim3(2048), dim3(256), 0, 0);
        hipLaunchKernelGGL(div_kernel, dim3(8192), dim3(256), 0, 0);
        err = hipGetLastError();
    }
    if (err == hipSuccess)
        err = hipDeviceSynchronize();
    if (err == hipSuccess)
        err = hipMemcpyFromSymbol(counts, HIP_SYMBOL(g_counts), sizeof zero);
    return (int)err;
}
