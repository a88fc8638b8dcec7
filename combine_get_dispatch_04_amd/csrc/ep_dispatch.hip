// ep_dispatch.hip -- token dispatch into the receive buffer ("DeepEP-Ascend"
// README, API Overview: dispatch and low_latency_dispatch; Quantization
// Modes in Normal Dispatch: bf16; float8_e4m3fn codes with float32 scales
// per 128 channels; INT8 dynamic and scalar FP8 with one float32 scale per
// token; MXFP8 (e4m3 or e5m2) and MXFP4 (e2m1) with a float8_e8m0fnu scale
// per 32 elements).
//
// Token-major: one block per (token, row segment).  The block reads its
// piece of x[t] once into registers (16 bytes = 8 channels per thread per
// piece), quantises it once, then computes the token's K receive rows from
// the layout tables, one slot per lane, and stores the piece to each of
// them (buffer stores bounded by the row), taking each slot into a scalar
// register with readlane.
//
// Quantisation groups map onto lanes: a 128-channel group is 16 consecutive
// lanes and a 32-channel MX block 4 lanes (8 and 2 when a lane holds two
// pieces), reduced with lane shuffles; a per-token scale is a block reduction
// when the row fits one block, and otherwise comes from a pre-pass kernel
// that takes each row's max into the workspace.  Scales are
// correctly rounded fp32 divisions.  Elements are divided by them with one
// reciprocal per scale and one correction step (codes equal to those of the
// correctly rounded quotient) or, for MX, scaled by the exact power of two
// 2^-E (a multiply for the fp8 widths, the conversion's scale operand for
// e2m1), then encoded to nearest even by gfx950's own conversion
// instructions.
#include "ep_common.h"
#include "ep_internal.h"

namespace ep {

namespace {

// num_dropped has a closed form: padded rows overflow by max(0, count - cap)
// per expert; contiguous rows by max(0, N - rows).
__device__ void write_num_dropped(const int32_t *offsets, int E, int padded, int cap_or_rows,
                                  int32_t *num_dropped)
{
    __shared__ int tmp[32];
    int d = 0;
    if (padded) {
        for (int e = threadIdx.x; e < E; e += blockDim.x) {
            int c = offsets[e + 1] - offsets[e];
            d += c > cap_or_rows ? c - cap_or_rows : 0;
        }
    } else if (threadIdx.x == 0) {
        int n = offsets[E];
        d = n > cap_or_rows ? n - cap_or_rows : 0;
    }
    int total;
    block_exclusive_scan(d, tmp, &total);
    if (threadIdx.x == 0)
        num_dropped[0] = total;
}

// With no tokens only the drop counter is written.
__global__ void dropped_only_kernel(const int32_t *__restrict__ offsets, int E, int padded,
                                    int cap_or_rows, int32_t *__restrict__ num_dropped)
{
    write_num_dropped(offsets, E, padded, cap_or_rows, num_dropped);
}

// n ints from global to shared memory by the whole block, 8 loads in flight
// per thread (one memory round trip per 8 * blockDim.x entries).
__device__ __forceinline__ void stage_ints(const int32_t *__restrict__ src, int n,
                                           int32_t *__restrict__ dst)
{
    for (int i0 = 0; i0 < n; i0 += 8 * blockDim.x) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x + threadIdx.x;
            v[u] = i < n ? src[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x + threadIdx.x;
            if (i < n)
                dst[i] = v[u];
        }
    }
}

// The one-launch low-latency form's per-expert results, from one block: an
// LDS histogram of all n entries gives the rows each expert received
// (capped at cap), the entries dropped for capacity, and the invalid ones.
__device__ void ll_counts(const int32_t *topk_idx, int n, int E, int cap, int32_t *ent,
                          int32_t *hist, int32_t *recv_count, int32_t *num_dropped,
                          int32_t *num_invalid)
{
    __shared__ int tmp[32];
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        hist[e] = 0;
    stage_ints(topk_idx, n, ent);
    __syncthreads();
    int inval = 0;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int v = ent[i];
        if ((unsigned)v < (unsigned)E)
            atomicAdd(&hist[v], 1);
        else if (v != -1)
            ++inval;
    }
    __syncthreads();
    int d = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = hist[e];
        recv_count[e] = c < cap ? c : cap;
        d += c > cap ? c - cap : 0;
    }
    int total;
    block_exclusive_scan(d, tmp, &total);
    if (threadIdx.x == 0)
        num_dropped[0] = total;
    block_exclusive_scan(inval, tmp, &total);
    if (threadIdx.x == 0)
        num_invalid[0] = total;
}

// The low-latency form with no tokens: every count is zero.
__global__ void ll_empty_kernel(int E, int32_t *__restrict__ recv_count,
                                int32_t *__restrict__ num_dropped,
                                int32_t *__restrict__ num_invalid)
{
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        recv_count[e] = 0;
    if (threadIdx.x == 0) {
        num_dropped[0] = 0;
        num_invalid[0] = 0;
    }
}

constexpr bool is_token_mode(int m) { return m == kQuantFp8Token || m == kQuantInt8Token; }
constexpr bool is_mx_mode(int m)
{
    return m == kQuantMxE4M3 || m == kQuantMxE5M2 || m == kQuantMxE2M1;
}
constexpr int mx_emax(int m) { return m == kQuantMxE4M3 ? 8 : (m == kQuantMxE5M2 ? 15 : 2); }

// Bytes of one receive row.
__host__ __device__ constexpr int64_t row_bytes(int m, int H)
{
    return m == kQuantBf16 ? 2 * (int64_t)H : (m == kQuantMxE2M1 ? H / 2 : (int64_t)H);
}

// Four int8 codes in one word, value i in byte i.
__device__ __forceinline__ uint32_t int8x4(float a, float b, float c, float d)
{
    return f32_to_int8_rne(a) | (f32_to_int8_rne(b) << 8) | (f32_to_int8_rne(c) << 16) |
           (f32_to_int8_rne(d) << 24);
}

// Max of v over the block (blockDim.x <= 256); every thread gets it.
__device__ __forceinline__ float block_max(float v)
{
    __shared__ float red[4];
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, kWave));
    const int wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
    if (threadIdx.x % kWave == 0)
        red[wave] = v;
    __syncthreads();
    float m = red[0];
    for (int w = 1; w < nw; ++w)
        m = fmaxf(m, red[w]);
    return m;
}

// Max |x| over one unit (U pieces of 8 bf16 channels).  |x| of a (non-NaN)
// bf16 orders like the integer of its low 15 bits, so it comes from the
// packed bits; a unit outside the row is zeros.
template <int U>
__device__ __forceinline__ float unit_amax(const u32x4 (&vj)[U])
{
    uint32_t m = 0u;
#pragma unroll
    for (int h = 0; h < U; ++h) {
        const uint32_t w[4] = {vj[h].x, vj[h].y, vj[h].z, vj[h].w};
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
    }
    return __uint_as_float(m << 16);
}

// A unit's max reduced over the lanes of its scale group: 16/U lanes hold a
// 128-channel group, 4/U lanes a 32-channel MX block (units and the lanes of
// a wave are multiples of these).
template <int MODE, int U>
__device__ __forceinline__ float group_amax(float a)
{
    if constexpr (MODE == kQuantFp8G128) {
#pragma unroll
        for (int o = 1; o < 16 / U; o <<= 1)
            a = fmaxf(a, __shfl_xor(a, o, kWave));
    } else if constexpr (is_mx_mode(MODE)) {
#pragma unroll
        for (int o = 1; o < 4 / U; o <<= 1)
            a = fmaxf(a, __shfl_xor(a, o, kWave));
    }
    return a;
}

// Lanes that share one scale (a power of two).
template <int MODE, int U>
__host__ __device__ constexpr int group_lanes()
{
    return MODE == kQuantFp8G128 ? 16 / U : (is_mx_mode(MODE) ? 4 / U : 1);
}

// Codes of one unit (8U bytes, or 4U for e2m1, in qj) and its group's
// scale (fp32 bits for the 128-channel and per-token scales, the e8m0 code
// for MX) from the group's max |x| `a`; per-token modes pass their scale.
template <int MODE, int U>
__device__ __forceinline__ void encode_unit(const u32x4 (&vj)[U], float a, float tok_scale,
                                            u32x4 &qj, uint32_t &scj)
{
    uint32_t wd[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < U; ++h) {
        const float f[8] = {bf16_lo(vj[h].x), bf16_hi(vj[h].x), bf16_lo(vj[h].y),
                            bf16_hi(vj[h].y), bf16_lo(vj[h].z), bf16_hi(vj[h].z),
                            bf16_lo(vj[h].w), bf16_hi(vj[h].w)};
        if constexpr (MODE == kQuantMxE2M1) {
            scj = (uint32_t)(mx_shared_exponent(a, 2) + 127);
            wd[h] = e2m1x8_scaled(f, scj);
            continue;
        }
        float g[8];
        if constexpr (is_mx_mode(MODE)) {
            const int e = mx_shared_exponent(a, mx_emax(MODE));
            // 2^-e as an fp32 pattern: e >= -127, and e <= 127 - emax for
            // finite bf16 input, so 127 - e lies in [2, 254]: a normal number
            const float m = __uint_as_float((uint32_t)(127 - e) << 23);
            // |x| * 2^-e < 2^(emax+1): bound it to the largest finite code
            constexpr float top = MODE == kQuantMxE4M3 ? 448.0f : 57344.0f;
            scj = (uint32_t)(e + 127);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                g[u] = __builtin_amdgcn_fmed3f(f[u] * m, -top, top);
        } else {
            // |x| <= a, so |x / s| <= 448 * (1 + 2^-23) < 464 (or 127.00002):
            // no bound needed before the e4m3 conversion
            const float s = MODE == kQuantFp8G128 ? (a == 0.0f ? 0.0f : a / 448.0f) : tok_scale;
            scj = __float_as_uint(s);
            if (s >= kFastDivMinScale) {
                const float r = 1.0f / s;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    g[u] = div_by_scale(f[u], s, r);
            } else {
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    g[u] = s == 0.0f ? 0.0f : f[u] / s;    // a zero group codes as 0
            }
        }
        if constexpr (MODE == kQuantInt8Token) {
            wd[2 * h] = int8x4(g[0], g[1], g[2], g[3]);
            wd[2 * h + 1] = int8x4(g[4], g[5], g[6], g[7]);
        } else if constexpr (MODE == kQuantMxE5M2) {
            wd[2 * h] = e5m2x4(g[0], g[1], g[2], g[3]);
            wd[2 * h + 1] = e5m2x4(g[4], g[5], g[6], g[7]);
        } else {
            wd[2 * h] = e4m3x4(g[0], g[1], g[2], g[3]);
            wd[2 * h + 1] = e4m3x4(g[4], g[5], g[6], g[7]);
        }
    }
    qj = u32x4{wd[0], wd[1], wd[2], wd[3]};
}

// Stores of one unit's codes and scale to receive row `s` (dst covers the
// row's codes).  i = the unit's index in the row; `lead` lanes hold the
// first unit of their scale group.
template <int MODE, int U>
__device__ __forceinline__ void store_unit(rsrc_t dst, int i, int units, int H, bool lead, int s,
                                           u32x4 qj, uint32_t scj, void *recv_s)
{
    if constexpr (MODE == kQuantMxE2M1) {
        if constexpr (U == 2)
            row_st8(dst, i * 8, u32x2{qj.x, qj.y});
        else
            row_st4(dst, i * 4, qj.x);
    } else {
        if constexpr (U == 2)
            row_st16(dst, i * 16, qj);
        else
            row_st8(dst, i * 8, u32x2{qj.x, qj.y});
    }
    if constexpr (MODE == kQuantFp8G128) {
        if (lead && i < units)
            reinterpret_cast<float *>(recv_s)[(size_t)s * (H >> 7) + i / (16 / U)] =
                __uint_as_float(scj);
    } else if constexpr (is_mx_mode(MODE)) {
        if (lead && i < units)
            reinterpret_cast<uint8_t *>(recv_s)[(size_t)s * (H >> 5) + i / (4 / U)] = (uint8_t)scj;
    }
}

// One block per (token, row segment).  A thread handles PPT units of U
// adjacent 16-byte pieces (U = 2 for the 8-bit codes when the row has an
// even number of pieces, so that a lane stores 16 bytes of codes).
//
// LL (the one-launch low-latency form, padded rows, K <= 64): there is no
// layout call.  Each block reads topk_idx up to its own token and ranks its
// token's entries itself: the rank of (t,k) is the number of entries before
// it in row-major order with the same expert, the same stable counting sort
// the layout performs.  One more block (grid.x = T + 1) writes the
// per-expert received counts, the dropped and the invalid counts (dynamic
// shared memory: that block's staged entries and histogram, or a token
// block's per-wave rank counts).
template <int PPT, int MODE, int U, bool LL>
__global__ void __launch_bounds__(256)
dispatch_kernel(const uint16_t *__restrict__ x, int H, const int32_t *__restrict__ topk_idx, int K,
                int E, const int32_t *__restrict__ offsets, int padded, int cap_or_rows, int CT, int CE,
                int nchunk, const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ local_rank,
                void *__restrict__ recv_x, void *__restrict__ recv_s,
                int32_t *__restrict__ slot_out, int32_t *__restrict__ recv_src,
                int32_t *__restrict__ num_dropped, const float *__restrict__ tok_amax,
                int32_t *__restrict__ recv_count, int32_t *__restrict__ num_invalid, int x_nt)
{
    constexpr bool QUANT = MODE != kQuantBf16;
    static_assert(U == 1 || (U == 2 && QUANT), "pairs are for the quantised modes");
    extern __shared__ int32_t ll_lds[];
    const int t = blockIdx.x;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int pieces = H >> 3;
    const int units = pieces / U;
    const int seg0 = blockIdx.y * PPT * bd;
    if constexpr (LL) {
        // the last block of the grid only counts (in parallel with the tokens)
        const int T = (int)gridDim.x - 1;
        if (t == T) {
            if (blockIdx.y == 0)
                ll_counts(topk_idx, T * K, E, cap_or_rows, ll_lds, ll_lds + T * K + 64,
                          recv_count, num_dropped, num_invalid);
            return;
        }
    } else if (t == 0 && blockIdx.y == 0) {
        write_num_dropped(offsets, E, padded, cap_or_rows, num_dropped);
    }

    // LL: the token's experts (lane k holds expert k) and the first pass of
    // earlier entries are requested before the row, so that the ranking
    // below waits for them and not for the row.
    int ll_e = -1;
    int ent0[4];
    if constexpr (LL) {
        const int row0 = t * K;
        ll_e = (tid & (kWave - 1)) < K ? topk_idx[row0 + (tid & (kWave - 1))] : -1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = u * bd + tid;
            ent0[u] = i < row0 + K - 1 ? topk_idx[i] : -1;
        }
    }

    // the row through a buffer descriptor: pieces past it read as zero with
    // no branch, so the loads are issued unconditionally and the waits for
    // the entries above can leave them in flight
    const rsrc_t xrow = row_rsrc(reinterpret_cast<const char *>(x) + (size_t)t * H * 2, H * 2);
    u32x4 v[PPT][U];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = seg0 + tid + j * bd;
#pragma unroll
        for (int h = 0; h < U; ++h)
            v[j][h] = x_nt ? row_ld16(xrow, (i * U + h) * 16)
                           : row_ld16_cached(xrow, (i * U + h) * 16);
    }

    // LL: lane k's rank (k < K <= 64), counted while the row is in flight.
    // Each thread holds the entries at its positions in registers (4 per
    // pass of 4 * blockDim.x entries, one coalesced round trip per pass);
    // for each of the token's experts every wave counts the matches among
    // the entries before (t,k) with ballots and popcounts and keeps the
    // count in lane k; one barrier then adds the waves' counts.  Lane k also
    // holds expert k of the token for the slot loop below.
    int ll_rank = 0;
    if constexpr (LL) {
        const int lane = tid & (kWave - 1), w = tid / kWave;
        const int row0 = t * K;
        int mine = 0;
        auto count_pass = [&](const int (&ent)[4], int i0) {
            for (int k = 0; k < K; ++k) {
                const int e = __builtin_amdgcn_readlane(ll_e, k);
                if ((unsigned)e >= (unsigned)E)
                    continue;
                const int lim = row0 + k;
                int cnt = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    cnt += __builtin_popcountll(ballot(ent[u] == e && i0 + u * bd + tid < lim));
                mine += lane == k ? cnt : 0;
            }
        };
        // a straight-line use of the entries: the wait for them here does not
        // wait for the row, which the compiler would otherwise flush before
        // the loop over k
        asm volatile("" ::"v"(ll_e), "v"(ent0[0]), "v"(ent0[1]), "v"(ent0[2]), "v"(ent0[3]));
        count_pass(ent0, 0);
        for (int i0 = 4 * bd; i0 < row0 + K - 1; i0 += 4 * bd) {
            int ent[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * bd + tid;
                ent[u] = i < row0 + K - 1 ? topk_idx[i] : -1;
            }
            count_pass(ent, i0);
        }
        int32_t *wcnt = ll_lds;                       // [waves][K]
        if (lane < K)
            wcnt[w * K + lane] = mine;
        __syncthreads();
        if (lane < K)
            for (int ww = 0; ww < bd / kWave; ++ww)
                ll_rank += wcnt[ww * K + lane];
    }

    // q: the unit's codes (8U bytes, or 4U for e2m1); sc: its group's scale
    // (fp32 bits for the 128-channel groups, the e8m0 code for MX)
    u32x4 q[QUANT ? PPT : 1];
    uint32_t sc[QUANT ? PPT : 1];
    float tok_scale = 0.0f;
    if constexpr (QUANT) {
        // channels are decoded to fp32 only where they are encoded (fewer
        // live registers)
        float amax[PPT];
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            amax[j] = unit_amax<U>(v[j]);
        if constexpr (is_token_mode(MODE)) {
            float a = 0.0f;
            if (tok_amax) {
                a = tok_amax[t];                      // a row over several blocks: taken before
            } else {
#pragma unroll
                for (int j = 0; j < PPT; ++j)
                    a = fmaxf(a, amax[j]);
                a = block_max(a);                     // the row is in this block: one segment
            }
#pragma unroll
            for (int j = 0; j < PPT; ++j)
                amax[j] = a;
            tok_scale = a == 0.0f ? 0.0f : a / (MODE == kQuantInt8Token ? 127.0f : 448.0f);
        }
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            encode_unit<MODE, U>(v[j], group_amax<MODE, U>(amax[j]), tok_scale, q[j], sc[j]);
            // keep the packed words here: left to itself the compiler sinks
            // the packing into the slot loop and keeps every code of every
            // unit live (131 VGPRs instead of about 60 at 7 pieces)
            asm volatile("" : "+v"(q[j]), "+v"(sc[j]));
        }
    }

    // The token's slots, 64 at a time, one per lane: its experts and ranks
    // are one coalesced load and the chunk bases one gather, instead of two
    // dependent scalar loads per slot.  Every wave computes them (the waves
    // of a block store the same slots); wave 0 of row segment 0 writes the
    // handle.  The stores then take each slot with readlane.
    const int c = t / CT;
    const int32_t *trow = topk_idx + (int64_t)t * K;
    const int32_t *rrow = LL ? nullptr : local_rank + (int64_t)t * K;
    const int64_t rb = row_bytes(MODE, H);
    const int lane = tid & (kWave - 1);
    const bool writer = blockIdx.y == 0 && tid < kWave;
    const bool lead = (tid & (group_lanes<MODE, U>() - 1)) == 0;
    for (int k0 = 0; k0 < K; k0 += kWave) {
        const int k = k0 + lane;
        int sl = -1;
        if (k < K) {
            const int e = LL ? ll_e : trow[k];                // LL: k == lane
            if ((unsigned)e < (unsigned)E) {
                int r;
                if constexpr (LL) {
                    r = ll_rank;                       // k == lane: K <= 64
                } else {
                    // rows longer than a layout chunk: each entry's own chunk
                    const int ck = CE > 0 ? (int)(((int64_t)t * K + k) / CE) : c;
                    r = chunk_base[(int64_t)e * nchunk + ck] + rrow[k];
                }
                if (padded)
                    sl = r < cap_or_rows ? e * cap_or_rows + r : -1;
                else {
                    sl = offsets[e] + r;
                    if (sl >= cap_or_rows)
                        sl = -1;
                }
            }
            if (writer) {
                slot_out[(int64_t)t * K + k] = sl;
                if (sl >= 0 && recv_src)
                    recv_src[sl] = t;
            }
        }
        const int kn = K - k0 < kWave ? K - k0 : kWave;
        for (int kk = 0; kk < kn; ++kk) {
            const int s = __builtin_amdgcn_readlane(sl, kk);
            if (s < 0)
                continue;
            const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(recv_x) + (size_t)s * rb, (int)rb);
            if constexpr (!QUANT) {
#pragma unroll
                for (int j = 0; j < PPT; ++j)
                    row_st16(dst, (seg0 + tid + j * bd) * 16, v[j][0]);
            } else {
#pragma unroll
                for (int j = 0; j < PPT; ++j)
                    store_unit<MODE, U>(dst, seg0 + tid + j * bd, units, H, lead, s, q[j], sc[j],
                                        recv_s);
                if constexpr (is_token_mode(MODE)) {
                    if (tid == 0 && blockIdx.y == 0)
                        reinterpret_cast<float *>(recv_s)[s] = tok_scale;
                }
            }
        }
    }
}

// Max |x| of each token's row (one block per token), for the per-token modes
// when a row spans several dispatch blocks.  The same packed-bits max as the
// dispatch itself, so the result is exact and equal to the one-block form.
__global__ void __launch_bounds__(256)
token_amax_kernel(const uint16_t *__restrict__ x, int H, float *__restrict__ tok_amax)
{
    const char *xrow = reinterpret_cast<const char *>(x) + (size_t)blockIdx.x * H * 2;
    float a = 0.0f;
    for (int i = threadIdx.x; i < (H >> 3); i += blockDim.x) {
        const u32x4 v[1] = {ld16(xrow + (size_t)i * 16)};
        a = fmaxf(a, unit_amax<1>(v));
    }
    a = block_max(a);
    if (threadIdx.x == 0)
        tok_amax[blockIdx.x] = a;
}

// Row pieces per thread and threads per block for a row of `pieces` 16-byte
// pieces: the block size (64..256) that wastes the fewest lanes, up to 8
// pieces per thread, and as many row segments (grid.y) as needed.
struct RowShape {
    int bd, ppt, nseg;
};

RowShape row_shape(int pieces, int maxppt = 8)
{
    RowShape best{64, 1, 1};
    long long best_waste = -1;
    for (int bd : {256, 128, 64}) {
        int ppt = (pieces + bd - 1) / bd;
        if (ppt < 1)
            ppt = 1;
        if (ppt > maxppt)
            ppt = maxppt;
        int nseg = (pieces + ppt * bd - 1) / (ppt * bd);
        if (nseg < 1)
            nseg = 1;
        long long waste = (long long)nseg * ppt * bd - pieces;
        if (best_waste < 0 || waste < best_waste) {
            best = {bd, ppt, nseg};
            best_waste = waste;
        }
    }
    return best;
}

template <int MODE, int U, bool LL>
hipError_t launch_dispatch_t(const LayoutPlan &p, const RowShape &rs, const uint16_t *x, int H,
                             const int32_t *topk_idx, const int32_t *offsets, int padded,
                             int cap_or_rows, void *recv_x, void *recv_s, int32_t *slot,
                             int32_t *recv_src, int32_t *num_dropped, const int32_t *hist,
                             const int32_t *rank, float *tamax_ws, int32_t *recv_count,
                             int32_t *num_invalid, size_t lds, int x_nt, hipStream_t s)
{
    // A per-token scale needs the whole row's max; when the row spans several
    // blocks it is taken first, into the workspace.
    float *tok_amax = nullptr;
    if (!LL && is_token_mode(MODE) && rs.nseg != 1) {
        tok_amax = tamax_ws;
        hipLaunchKernelGGL(token_amax_kernel, dim3(p.T), dim3(256), 0, s, x, H, tok_amax);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    if ((uint64_t)p.T * rs.bd > 0xFFFFFFFFull)    // work-items per grid dimension fit 32 bits
        return hipErrorInvalidConfiguration;
    dim3 grid(p.T + (LL ? 1 : 0), rs.nseg), block(rs.bd);
#define EP_DISPATCH_CASE(N)                                                                      \
    case N:                                                                                      \
        hipLaunchKernelGGL((dispatch_kernel<N, MODE, U, LL>), grid, block, lds, s, x, H,         \
                           topk_idx, p.K, p.E, offsets, padded, cap_or_rows, p.CT, p.CE,         \
                           p.nchunk,                                                             \
                           hist, rank, recv_x, recv_s, slot, recv_src, num_dropped, tok_amax,    \
                           recv_count, num_invalid, x_nt);                                       \
        break;
    if constexpr (LL) {          // at most 2 units per thread (launch_ll_dispatch)
        switch (rs.ppt) {
            EP_DISPATCH_CASE(1)
            EP_DISPATCH_CASE(2)
        default:
            return hipErrorInvalidValue;
        }
    } else {
        switch (rs.ppt) {
            EP_DISPATCH_CASE(1)
            EP_DISPATCH_CASE(2)
            EP_DISPATCH_CASE(3)
            EP_DISPATCH_CASE(4)
            EP_DISPATCH_CASE(5)
            EP_DISPATCH_CASE(6)
            EP_DISPATCH_CASE(7)
            EP_DISPATCH_CASE(8)
        default:
            return hipErrorInvalidValue;
        }
    }
#undef EP_DISPATCH_CASE
    return hipGetLastError();
}

// Units per row: 8-bit codes of rows with an even number of pieces go in
// pairs of pieces (16-byte stores; measured at prefill: fp8 per 128 channels
// 63 -> 56 us, MXFP8 71 -> 54 us); e2m1 stays at one piece (4-byte stores
// measured faster than 8-byte ones there: 31 vs 33 us).
bool pairs_for(int quant, int H)
{
    return quant != kQuantBf16 && quant != kQuantMxE2M1 && (H / 8) % 2 == 0;
}

// The low-latency form's block shape: 256 threads, at most 2 units per
// thread, as few row segments as that allows (each segment's block repeats
// the token's ranking, which 256 threads share); a per-token row must fit
// one block (nseg = 0: too long).  Measured at decode (T = 128, H = 7168):
// bf16 rows (896 units) over 7 one-wave blocks took 13.4 us for the
// dispatch (events), over 2 blocks of 256 threads 10.3 us.
// The low-latency launch: 256 threads per block and, outside the per-token
// modes, one unit per thread while the token blocks stay within one per CU
// (256 on MI355X), else two.  At decode (T = 128, H = 7168) the fp8 and
// MXFP8 codes then take two blocks per token instead of one, which halves
// each block's encode and store issue (one wave per SIMD: the work is a
// dependent instruction chain, not bandwidth): step 9.9-10.2 -> 9.5-10.0 us
// (fp8, 128-channel scales; means of five runs 10.06 -> 9.72), 9.8-10.0 ->
// 9.3-9.9 (MXFP8).  bf16 with four blocks per token (512 in all) was slower,
// 12.0 -> 14.4 us, and keeps two units.
constexpr int64_t kLlBlocks = 256;

RowShape ll_shape(int quant, int H, int T)
{
    const int units = pairs_for(quant, H) ? H / 16 : H / 8;
    if (is_token_mode(quant)) {
        // the row's max is a block reduction: the row stays in one block
        if (units > 2 * 256)
            return {256, 2, 0};
        return {256, units <= 256 ? 1 : 2, 1};
    }
    const int n1 = (units + 255) / 256;
    if ((int64_t)T * n1 <= kLlBlocks)
        return {256, 1, n1};
    return {256, 2, (units + 511) / 512};
}

}  // namespace

// Launch of the dispatch kernel for one mode, with or without pairs of
// pieces per unit.
#define EP_MODE_SWITCH(LL, ...)                                                                  \
    do {                                                                                         \
        if (!pairs) {                                                                            \
            switch (quant) {                                                                     \
            case kQuantBf16: return launch_dispatch_t<kQuantBf16, 1, LL>(__VA_ARGS__);           \
            case kQuantFp8G128: return launch_dispatch_t<kQuantFp8G128, 1, LL>(__VA_ARGS__);     \
            case kQuantFp8Token: return launch_dispatch_t<kQuantFp8Token, 1, LL>(__VA_ARGS__);   \
            case kQuantInt8Token: return launch_dispatch_t<kQuantInt8Token, 1, LL>(__VA_ARGS__); \
            case kQuantMxE4M3: return launch_dispatch_t<kQuantMxE4M3, 1, LL>(__VA_ARGS__);       \
            case kQuantMxE5M2: return launch_dispatch_t<kQuantMxE5M2, 1, LL>(__VA_ARGS__);       \
            case kQuantMxE2M1: return launch_dispatch_t<kQuantMxE2M1, 1, LL>(__VA_ARGS__);       \
            default: return hipErrorInvalidValue;                                                \
            }                                                                                    \
        }                                                                                        \
        switch (quant) {                                                                         \
        case kQuantFp8G128: return launch_dispatch_t<kQuantFp8G128, 2, LL>(__VA_ARGS__);         \
        case kQuantFp8Token: return launch_dispatch_t<kQuantFp8Token, 2, LL>(__VA_ARGS__);       \
        case kQuantInt8Token: return launch_dispatch_t<kQuantInt8Token, 2, LL>(__VA_ARGS__);     \
        case kQuantMxE4M3: return launch_dispatch_t<kQuantMxE4M3, 2, LL>(__VA_ARGS__);           \
        case kQuantMxE5M2: return launch_dispatch_t<kQuantMxE5M2, 2, LL>(__VA_ARGS__);           \
        default: return hipErrorInvalidValue;                                                    \
        }                                                                                        \
    } while (0)

hipError_t launch_dispatch(const LayoutPlan &p, const uint16_t *x, int H, const int32_t *topk_idx,
                           const int32_t *offsets, bool padded, int cap_or_rows, int quant,
                           void *recv_x, void *recv_scales, int32_t *slot, int32_t *recv_src,
                           int32_t *num_dropped, char *ws, hipStream_t s)
{
    const int32_t *hist = reinterpret_cast<const int32_t *>(ws + p.off_hist);
    const int32_t *rank = reinterpret_cast<const int32_t *>(ws + p.off_rank);
    float *tamax = reinterpret_cast<float *>(ws + p.off_tamax);
    if (p.T == 0) {
        hipLaunchKernelGGL(dropped_only_kernel, dim3(1), dim3(256), 0, s, offsets, p.E,
                           (int)padded, cap_or_rows, num_dropped);
        return hipGetLastError();
    }
    const bool pairs = pairs_for(quant, H);
    // Few tokens (a latency-bound launch): at most 2 units per thread, so a
    // row spreads over more threads.  Measured at decode (T = 128, H = 7168):
    // fp8 per 128 channels 20.6 -> 10.4 us, MXFP8 15.8 -> 9.6 us, bf16 about
    // the same.  A per-token row must stay in one block.
    const int units = pairs ? H / 16 : H / 8;
    RowShape rs = row_shape(units, p.T < 1024 ? 2 : 8);
    if (is_token_mode(quant) && rs.nseg != 1)
        rs = row_shape(units, 8);
    // The 8-bit codes of many tokens: x rows read non-temporally, so that x
    // does not take the memory-side cache (MALL) the written codes fit in.
    // Measured at prefill (T = 4096, 242 MB of codes and scales, steps by
    // wall clock, two A/B runs each): fp8 128-channel 171.0 -> 157.6 us,
    // per-token fp8 166.7 -> 155.1, int8 166.5 -> 154.9, MXFP8 170.3 ->
    // 157.3 / 170.0 -> 157.3; MXFP4 (125 MB) 130.7 -> 133.0, bf16 (470 MB)
    // 182.6 -> 183.4, decode with the pair (T = 128) no gain: cached there.
    // bf16 rows from a large source (a receiving rank's packed rows: 341 MB
    // at prefill with 8 ranks) are read non-temporally too while the rows
    // written stay within a few MALL sizes.  The rank share's step at
    // prefill: R = 8 571.7-571.9 -> 563.5 us, R = 32 641.5 -> 629.9; with
    // rows far beyond the MALL (3.4 GB or more: the large workload, alone
    // or as one rank's share) the default policy was 2-10 us faster.
    const size_t x_bytes = (size_t)p.T * H * 2;
    const size_t rows_bytes =
        (size_t)(padded ? (int64_t)p.E * cap_or_rows : (int64_t)cap_or_rows) * H * 2;
    const int x_nt = (quant != kQuantBf16 && quant != kQuantMxE2M1 && p.T >= 1024) ||
                     (quant == kQuantBf16 && x_bytes > ((size_t)128 << 20) &&
                      rows_bytes <= ((size_t)1 << 30));
    EP_MODE_SWITCH(false, p, rs, x, H, topk_idx, offsets, (int)padded, cap_or_rows, recv_x,
                   recv_scales, slot, recv_src, num_dropped, hist, rank, tamax, nullptr, nullptr,
                   0, x_nt, s);
}

bool ll_dispatch_fits(int T, int K, int H, int quant)
{
    return (int64_t)T * K <= kLlMaxEntries && K <= kLlMaxTopk && ll_shape(quant, H, T).nseg > 0;
}

hipError_t launch_ll_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx, int K,
                              int E, int cap, int quant, void *recv_x, void *recv_scales,
                              int32_t *slot, int32_t *recv_src, int32_t *recv_count,
                              int32_t *num_dropped, int32_t *num_invalid, hipStream_t s)
{
    if (!ll_dispatch_fits(T, K, H, quant))
        return hipErrorInvalidValue;
    if (T == 0) {
        hipLaunchKernelGGL(ll_empty_kernel, dim3(1), dim3(256), 0, s, E, recv_count, num_dropped,
                           num_invalid);
        return hipGetLastError();
    }
    // no chunk tables: one chunk, ranks found in the kernel
    LayoutPlan p{};
    p.T = T;
    p.K = K;
    p.E = E;
    p.R = 1;
    p.CT = T;
    p.nchunk = 1;
    const bool pairs = pairs_for(quant, H);
    const RowShape rs = ll_shape(quant, H, T);
    // the count block's staged entries and histogram; the token blocks' rank
    // counts per wave (4 waves x K)
    const size_t lds = std::max<size_t>((size_t)T * K + 64 + E, 4 * 64) * sizeof(int32_t);
    EP_MODE_SWITCH(true, p, rs, x, H, topk_idx, nullptr, 1, cap, recv_x, recv_scales, slot,
                   recv_src, num_dropped, nullptr, nullptr, nullptr, recv_count, num_invalid, lds,
                   0, s);
}
#undef EP_MODE_SWITCH

}  // namespace ep
