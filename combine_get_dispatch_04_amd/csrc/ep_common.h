// ep_common.h -- device helpers shared by the libep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- memory
// 16-byte row pieces.  Streams that are written once and not read again by
// the same kernel use non-temporal stores so they do not displace inputs
// that are still being read from the caches.
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ u32x4 ld16_nt(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
__device__ __forceinline__ void st16_nt(void *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void st8_nt(void *p, u32x2 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

// Buffer (V#) accesses with an explicit cache policy.  A descriptor covers
// one row (base = the row, num_records = its bytes), so pieces past the row
// end read as zero and are not written.  Policy bits of gfx950 buffer
// instructions: bit 0 = sc0, bit 1 = nt, bit 4 = sc1.  Measured on the
// prefill workload: receive-row stores with sc1 and row loads with nt were
// the fastest of the eight combinations each (dispatch 80 vs 95 us with nt
// stores; combine 93 vs 147 us with plain loads).
constexpr int kBufferDword3 = 0x00020000;     // raw 32-bit data format
constexpr int kStorePolicy = 16;              // sc1
constexpr int kLoadPolicy = 2;                // nt
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t row_rsrc(const void *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, kBufferDword3);
}
__device__ __forceinline__ void row_st16(rsrc_t r, int off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kStorePolicy);
}
__device__ __forceinline__ void row_st8(rsrc_t r, int off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kStorePolicy);
}
__device__ __forceinline__ void row_st4(rsrc_t r, int off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kStorePolicy);
}
__device__ __forceinline__ u32x4 row_ld16(rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kLoadPolicy);
}
__device__ __forceinline__ u32x2 row_ld8(rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kLoadPolicy);
}
// Default policy, for rows that other blocks read again.
__device__ __forceinline__ u32x4 row_ld16_cached(rsrc_t r, int off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs): add half an ulp
// of the kept part minus one, plus the kept part's lowest bit, then truncate.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------- fp8 / fp4
// gfx950 converts fp32 to the OCP 8-bit formats (E4M3: bias 7, largest
// finite 448, no infinity; E5M2: bias 15, largest finite 57344) and to E2M1
// in hardware, rounding to nearest even and keeping the sign of zero.  On
// every finite fp32 input these instructions give the same code as a
// software round-to-nearest-even encoder, with two exceptions that callers
// avoid: the plain fp8 conversions do not saturate (|v| >= 464 for E4M3,
// >= 61440 for E5M2 give a NaN code), so an input that may reach them is
// first bounded with med3 to the largest finite value, which rounds the same
// way.  The E2M1 conversion saturates at 6 by itself.
//
// Four fp8 codes in one word, value i in byte i.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d)
{
    const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
__device__ __forceinline__ uint32_t e5m2x4(float a, float b, float c, float d)
{
    const uint32_t w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0u, false);
    return __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
}
// Eight E2M1 codes of v[i] * 2^-E in one word, value 2i in the low nibble of
// byte i and 2i+1 in the high nibble.  The scaled conversion reads only the
// exponent field of its scale operand, so `e8m0` (= E + 127, 0..254) is
// passed as that field: E = -127 gives the pattern of +0.0, which the
// instruction takes as 2^-127.
__device__ __forceinline__ uint32_t e2m1x8_scaled(const float (&v)[8], uint32_t e8m0)
{
    const float scale = __uint_as_float(e8m0 << 23);
    uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], scale, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], scale, 3);
}

// ---------------------------------------------------------------- x / s
// Division by a scale shared by many elements, with one reciprocal per
// scale: r = RN(1/s), q0 = RN(x*r), the remainder x - s*q0 exactly (one
// fma), q = RN(q0 + rem*r).  By Markstein's theorem (r correctly rounded,
// q0 within one ulp) q is the correctly rounded quotient as long as the
// remainder does not underflow.  With s >= 2^-64 that holds for every
// quotient of magnitude 2^-11 or more; smaller quotients may be off in the
// last place, but every E4M3 or int8 code of a quantity below 2^-11 is a
// zero code either way, so the codes equal those of x / s.  The final copysign keeps
// -0 (the fma sum of +0 and -0 is +0).  Checked for every pair of bf16
// |x| <= amax with s = amax/448 and s = amax/127.
constexpr float kFastDivMinScale = 0x1p-64f;
__device__ __forceinline__ float div_by_scale(float x, float s, float r)
{
    const float q0 = x * r;
    const float rem = fmaf(-q0, s, x);
    return __builtin_copysignf(fmaf(rem, r, q0), x);
}

// fp32 -> int8 code (two's complement byte): round to nearest even, clamped
// to [-127, 127].
__device__ __forceinline__ uint32_t f32_to_int8_rne(float v)
{
    float r = fminf(fmaxf(__builtin_rintf(v), -127.0f), 127.0f);
    return (uint32_t)(int)r & 0xFFu;
}

// Shared exponent of a 32-element MX block: floor(log2(amax)) - emax,
// clamped to [-127, 127]; an all-zero block gives -127.  floor(log2) is the
// exponent field, or for an fp32 subnormal the position of the top bit.
__device__ __forceinline__ int mx_shared_exponent(float amax, int emax)
{
    const uint32_t a = __float_as_uint(amax);
    if (a == 0u)
        return -127;
    int e = (a >> 23) ? (int)(a >> 23) - 127 : (31 - (int)__clz(a)) - 149;
    e -= emax;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ---------------------------------------------------------------- waves
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t lanemask_lt(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}
// Number of set bits of m in lanes below mine (mbcnt).
__device__ __forceinline__ int lanes_below(uint64_t m)
{
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Lanes of this wave whose `key` equals mine, among lanes where `active`
// holds.  gfx950 has no match instruction: one ballot per key bit narrows
// the set.  Must be called by all lanes of the wave (converged).
__device__ __forceinline__ uint64_t match_key(int key, bool active, int nbits)
{
    uint64_t m = ballot(active);
    for (int b = 0; b < nbits; ++b) {
        bool bit = (key >> b) & 1;
        uint64_t bb = ballot(active && bit);
        m &= bit ? bb : ~bb;
    }
    return active ? m : 0ull;
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP row shifts
// (Hillis-Steele inside each 16-lane row), then row broadcasts of lane 15
// into rows 1 and 3 and of lane 31 into rows 2 and 3.  Lanes whose DPP
// source falls outside the row add 0.
__device__ __forceinline__ int wave_inclusive_scan(int v, int /*lane*/)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_sum(int v)
{
    return __builtin_amdgcn_readlane(wave_inclusive_scan(v, 0), kWave - 1);
}

// Exclusive prefix sum over a block's threads (blockDim.x <= 1024, multiple
// of 64).  `tmp` holds >= 17 ints of shared memory.  Returns my exclusive
// prefix; *total receives the block sum.  All threads must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp, int *total)
{
    int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    int nw = blockDim.x / kWave;
    int inc = wave_inclusive_scan(v, lane);
    if (lane == kWave - 1)
        tmp[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int s = lane < nw ? tmp[lane] : 0;
        int si = wave_inclusive_scan(s, lane);
        if (lane < nw)
            tmp[lane] = si - s;
        if (lane == kWave - 1)
            tmp[16] = si;
    }
    __syncthreads();
    int ex = tmp[wave] + inc - v;
    *total = tmp[16];
    __syncthreads();
    return ex;
}

}  // namespace ep
