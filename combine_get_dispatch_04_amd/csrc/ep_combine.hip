// ep_combine.hip -- weighted gather-reduce back to token order.
//   Token choice ("DeepEP-Ascend" README, API Overview: combine through the
//   dispatch handle; low_latency_combine also takes topk_weights):
//     out[t] = bf16( sum_k w[t,k] * y[slot[t,k]] )
//   Expert choice ("[Feature Request] Support Expert-Choice Routing via
//   Native Expert-Centric API", Solution 1: weights with the expert-centric
//   indices):
//     out[t] = bf16( sum over token t's entries j of w[j] * y[j] )
//
// One block per (token, row segment); each thread owns PPT 16-byte pieces
// (8 channels each) and keeps 8*PPT fp32 accumulators.  Source rows are
// block-uniform: their indices and weights live in scalar registers (scalar
// loads, or one vector load of 64 slots and readlane in the batched form).
// Each thread loads its pieces of a row with non-temporal buffer loads (each
// y row is read once) and accumulates with fp32 FMAs in ascending k / entry
// order, then rounds once to bf16 (nearest even).  A token with no source
// row writes +0.
//
// The receiving rank of the expert-parallel exchange sums the same way into
// fp32 rows (partial_kernel): its partial sums per received row travel back
// to the sender, which adds them over ranks (ep_rank.hip).
#include "ep_common.h"
#include "ep_internal.h"

namespace ep {

namespace {

template <int PPT>
__device__ __forceinline__ void acc_row(float (&acc)[PPT][8], const char *src, float wk, int seg0,
                                        int pieces)
{
    const rsrc_t row = row_rsrc(src, pieces * 16);     // pieces past the row read as zero
    u32x4 v[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j)
        v[j] = row_ld16(row, (seg0 + threadIdx.x + j * blockDim.x) * 16);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        acc[j][0] = fmaf(wk, bf16_lo(v[j].x), acc[j][0]);
        acc[j][1] = fmaf(wk, bf16_hi(v[j].x), acc[j][1]);
        acc[j][2] = fmaf(wk, bf16_lo(v[j].y), acc[j][2]);
        acc[j][3] = fmaf(wk, bf16_hi(v[j].y), acc[j][3]);
        acc[j][4] = fmaf(wk, bf16_lo(v[j].z), acc[j][4]);
        acc[j][5] = fmaf(wk, bf16_hi(v[j].z), acc[j][5]);
        acc[j][6] = fmaf(wk, bf16_lo(v[j].w), acc[j][6]);
        acc[j][7] = fmaf(wk, bf16_hi(v[j].w), acc[j][7]);
    }
}

// bf16 rows: 16 bytes per 8 channels, stored with the receive rows' policy
// (sc1).  Measured in the step against plain stores (two A/B runs each):
// large 1334.6-1335.6 -> 1324.9-1327.3 us, fp8 prefill 156.6-156.7 ->
// 154.1-154.4, rounds of 1024 177.2-177.5 -> 175.0-175.1, bf16 prefill
// 182.6-182.9 -> 182.9-183.2.  (Non-temporal stores: fp8 prefill 147.2, but
// bf16 prefill 190.2-191.3 and large 1349-1350.)
template <int PPT>
__device__ __forceinline__ void store_row(const float (&acc)[PPT][8], uint16_t *out, int H, int t,
                                          int seg0, int pieces)
{
    const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(out) + (size_t)t * H * 2, pieces * 16);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        int i = seg0 + threadIdx.x + j * blockDim.x;
        if (i < pieces) {
            u32x4 o;
            o.x = pack_bf16x2(acc[j][0], acc[j][1]);
            o.y = pack_bf16x2(acc[j][2], acc[j][3]);
            o.z = pack_bf16x2(acc[j][4], acc[j][5]);
            o.w = pack_bf16x2(acc[j][6], acc[j][7]);
            row_st16(dst, i * 16, o);
        }
    }
}

// G == 1: one source row per round, its slot and weight scalar loads; slots
// outside [0, y_rows) are skipped.  G > 1: G valid source rows per round,
// all G*PPT row pieces requested before the first FMA.
template <int PPT, int G>
__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t *__restrict__ y, int y_rows, int H,
               const int32_t *__restrict__ slot, const float *__restrict__ w, int K,
               uint16_t *__restrict__ out)
{
    const int t = blockIdx.x;
    const int pieces = H >> 3;
    const int seg0 = blockIdx.y * PPT * blockDim.x;
    float acc[PPT][8];
#pragma unroll
    for (int j = 0; j < PPT; ++j)
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc[j][u] = 0.0f;
    const int32_t *srow = slot + (int64_t)t * K;
    const float *wrow = w ? w + (int64_t)t * K : nullptr;
    if constexpr (G == 1) {
        for (int k = 0; k < K; ++k) {
            const int s = srow[k];
            if ((unsigned)s >= (unsigned)y_rows)
                continue;
            const float wk = wrow ? wrow[k] : 1.0f;
            acc_row<PPT>(acc, reinterpret_cast<const char *>(y) + (size_t)s * H * 2, wk, seg0,
                         pieces);
        }
    } else {
        // Each round takes the next G valid slots in ascending k, so padding
        // and dropped slots cost no round trip: every wave loads 64 of the
        // token's slots at once (one per lane; all waves of the block load
        // the same ones), a ballot marks the valid ones, and each round reads
        // its slots and weights out of that mask with readlane.
        const int lane = threadIdx.x & (kWave - 1);
        for (int k0 = 0; k0 < K; k0 += kWave) {
            const int kk = k0 + lane;
            const int sv = kk < K ? srow[kk] : -1;
            const bool valid = (unsigned)sv < (unsigned)y_rows;
            const float wv = valid ? (wrow ? wrow[kk] : 1.0f) : 0.0f;
            uint64_t m = ballot(valid);
            while (m) {
                int sel[G];
                float wk[G];
                bool ok[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    ok[g] = m != 0;
                    const int b = ok[g] ? (int)__builtin_ctzll(m) : 0;
                    m &= m - 1;
                    sel[g] = ok[g] ? __builtin_amdgcn_readlane(sv, b) : 0;
                    wk[g] = ok[g] ? __int_as_float(
                                        __builtin_amdgcn_readlane(__float_as_int(wv), b))
                                  : 0.0f;
                }
                u32x4 v[G][PPT];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const rsrc_t src = row_rsrc(reinterpret_cast<const char *>(y) +
                                                    (size_t)sel[g] * H * 2,
                                                ok[g] ? pieces * 16 : 0);
#pragma unroll
                    for (int j = 0; j < PPT; ++j)
                        v[g][j] = row_ld16(src, (seg0 + threadIdx.x + j * blockDim.x) * 16);
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if (!ok[g])
                        continue;
#pragma unroll
                    for (int j = 0; j < PPT; ++j) {
                        acc[j][0] = fmaf(wk[g], bf16_lo(v[g][j].x), acc[j][0]);
                        acc[j][1] = fmaf(wk[g], bf16_hi(v[g][j].x), acc[j][1]);
                        acc[j][2] = fmaf(wk[g], bf16_lo(v[g][j].y), acc[j][2]);
                        acc[j][3] = fmaf(wk[g], bf16_hi(v[g][j].y), acc[j][3]);
                        acc[j][4] = fmaf(wk[g], bf16_lo(v[g][j].z), acc[j][4]);
                        acc[j][5] = fmaf(wk[g], bf16_hi(v[g][j].z), acc[j][5]);
                        acc[j][6] = fmaf(wk[g], bf16_lo(v[g][j].w), acc[j][6]);
                        acc[j][7] = fmaf(wk[g], bf16_hi(v[g][j].w), acc[j][7]);
                    }
                }
            }
        }
    }
    store_row<PPT>(acc, out, H, t, seg0, pieces);
}

// The receiving rank's partial sums: fp32 output rows.  A unit is 4
// channels (8 bytes of y, 16 bytes of output), so that each store
// instruction of a wave writes 1 KiB of a row with no gaps.  Each round takes
// the row's next G valid slots in ascending k (one load of 64 slots per wave,
// a ballot, readlane), requests all of their pieces, then adds them in order
// with fp32 FMAs.
template <int PPT, int G>
__global__ void __launch_bounds__(256)
partial_kernel(const uint16_t *__restrict__ y, int y_rows, int H,
               const int32_t *__restrict__ slot, const float *__restrict__ w, int K,
               float *__restrict__ out)
{
    const int t = blockIdx.x;
    const int units = H >> 2;
    const int seg0 = blockIdx.y * PPT * blockDim.x;
    const int lane = threadIdx.x & (kWave - 1);
    float acc[PPT][4];
#pragma unroll
    for (int j = 0; j < PPT; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc[j][u] = 0.0f;
    const int32_t *srow = slot + (int64_t)t * K;
    const float *wrow = w ? w + (int64_t)t * K : nullptr;
    for (int k0 = 0; k0 < K; k0 += kWave) {
        const int kk = k0 + lane;
        const int sv = kk < K ? srow[kk] : -1;
        const bool valid = (unsigned)sv < (unsigned)y_rows;
        const float wv = valid ? (wrow ? wrow[kk] : 1.0f) : 0.0f;
        uint64_t m = ballot(valid);
        while (m) {
            int sel[G];
            float wk[G];
            bool ok[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                ok[g] = m != 0;
                const int b = ok[g] ? (int)__builtin_ctzll(m) : 0;
                m &= m - 1;
                sel[g] = ok[g] ? __builtin_amdgcn_readlane(sv, b) : 0;
                wk[g] = ok[g] ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), b))
                              : 0.0f;
            }
            u32x2 v[G][PPT];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const rsrc_t src = row_rsrc(reinterpret_cast<const char *>(y) +
                                                (size_t)sel[g] * H * 2,
                                            ok[g] ? units * 8 : 0);
#pragma unroll
                for (int j = 0; j < PPT; ++j)
                    v[g][j] = row_ld8(src, (seg0 + threadIdx.x + j * blockDim.x) * 8);
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (!ok[g])
                    continue;
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    acc[j][0] = fmaf(wk[g], bf16_lo(v[g][j].x), acc[j][0]);
                    acc[j][1] = fmaf(wk[g], bf16_hi(v[g][j].x), acc[j][1]);
                    acc[j][2] = fmaf(wk[g], bf16_lo(v[g][j].y), acc[j][2]);
                    acc[j][3] = fmaf(wk[g], bf16_hi(v[g][j].y), acc[j][3]);
                }
            }
        }
    }
    // sc1 stores, as for the bf16 rows: the rank share's step (R = 8) went
    // from 576.6-578.0 to 568.8-569.6 us, this kernel 194.0-194.3 -> 188.3-188.6
    const rsrc_t dst = row_rsrc(out + (size_t)t * H, units * 16);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = seg0 + threadIdx.x + j * blockDim.x;
        if (i < units)
            row_st16(dst, i * 16, u32x4{__float_as_uint(acc[j][0]), __float_as_uint(acc[j][1]),
                                        __float_as_uint(acc[j][2]), __float_as_uint(acc[j][3])});
    }
}

// G entries per round: their row indices and weights are scalar loads, then
// all G*PPT row pieces are requested before the first FMA, so a token that
// many experts picked waits on ceil(m/G) memory round trips, not m.
template <int PPT, int G>
__global__ void __launch_bounds__(256)
ec_combine_kernel(const uint16_t *__restrict__ y, const float *__restrict__ w, int n_ent, int H,
                  const int32_t *__restrict__ tok_off, const int32_t *__restrict__ tok_ent,
                  uint16_t *__restrict__ out)
{
    const int t = blockIdx.x;
    const int pieces = H >> 3;
    const int seg0 = blockIdx.y * PPT * blockDim.x;
    float acc[PPT][8];
#pragma unroll
    for (int k = 0; k < PPT; ++k)
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc[k][u] = 0.0f;
    const int b = tok_off[t], e = tok_off[t + 1];
    const int n = (b >= 0 && e >= b && e <= n_ent) ? e - b : 0;
    for (int a0 = 0; a0 < n; a0 += G) {
        bool ok[G];
        float wk[G];
        u32x4 v[G][PPT];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int j = a0 + g < n ? tok_ent[b + a0 + g] : -1;
            ok[g] = (unsigned)j < (unsigned)n_ent;
            const size_t row = ok[g] ? (size_t)j : 0;
            wk[g] = ok[g] ? w[row] : 0.0f;
            // an entry that is not used gets a zero-length descriptor: no access
            const rsrc_t src = row_rsrc(reinterpret_cast<const char *>(y) + row * H * 2,
                                        ok[g] ? pieces * 16 : 0);
#pragma unroll
            for (int k = 0; k < PPT; ++k)
                v[g][k] = row_ld16(src, (seg0 + threadIdx.x + k * blockDim.x) * 16);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (!ok[g])
                continue;
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                acc[k][0] = fmaf(wk[g], bf16_lo(v[g][k].x), acc[k][0]);
                acc[k][1] = fmaf(wk[g], bf16_hi(v[g][k].x), acc[k][1]);
                acc[k][2] = fmaf(wk[g], bf16_lo(v[g][k].y), acc[k][2]);
                acc[k][3] = fmaf(wk[g], bf16_hi(v[g][k].y), acc[k][3]);
                acc[k][4] = fmaf(wk[g], bf16_lo(v[g][k].z), acc[k][4]);
                acc[k][5] = fmaf(wk[g], bf16_hi(v[g][k].z), acc[k][5]);
                acc[k][6] = fmaf(wk[g], bf16_lo(v[g][k].w), acc[k][6]);
                acc[k][7] = fmaf(wk[g], bf16_hi(v[g][k].w), acc[k][7]);
            }
        }
    }
    store_row<PPT>(acc, out, H, t, seg0, pieces);
}

struct RowShape {
    int bd, ppt, nseg;
};

// Fewest idle lanes over block sizes 256/128/64 with at most `maxppt`
// pieces per thread; more row segments (grid.y) when a row is longer.
RowShape row_shape(int pieces, int maxppt)
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

}  // namespace

#define EP_PPT_SWITCH(PPT_VAR, CASE) \
    switch (PPT_VAR) {               \
        CASE(1)                      \
        CASE(2)                      \
        CASE(3)                      \
        CASE(4)                      \
        CASE(5)                      \
        CASE(6)                      \
        CASE(7)                      \
        CASE(8)                      \
    default:                         \
        return hipErrorInvalidValue; \
    }

hipError_t launch_combine(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                          const float *w, int T, int K, uint16_t *out, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    // Many source rows per token (K >= 12), or few tokens (T < 1024, where
    // the grid does not fill the chip and each row's round trips are the
    // time): at most 2 pieces per thread, so a row spreads over more blocks,
    // and 4 rows requested per round.  Measured on T=16384, K=16 (3.2 GB of
    // rows): 683 -> 641 us; on T=128, K=8: 10.2 -> 9.2 us.  At K = 8 and
    // T = 4096 that shape was 4 us slower than 7 pieces per thread, one row
    // per round.  Few tokens with K < 12 (decode): one piece per thread and
    // 8 rows per round, so a token's K = 8 rows are one round trip (decode
    // combine 7.0-7.1 -> 6.75 us by events, in two runs each).
    const bool many = K >= 12 || T < 1024;
    const bool few = T < 1024 && K < 12;
    RowShape rs = row_shape(H / 8, few ? 1 : (many ? 2 : 8));
    if ((uint64_t)T * rs.bd > 0xFFFFFFFFull)      // work-items per grid dimension fit 32 bits
        return hipErrorInvalidConfiguration;
    dim3 grid(T, rs.nseg), block(rs.bd);
    if (few) {
        hipLaunchKernelGGL((combine_kernel<1, 8>), grid, block, 0, s, y, y_rows, H, slot, w,
                           K, out);
        return hipGetLastError();
    }
#define EP_COMBINE_CASE(N)                                                                       \
    case N:                                                                                      \
        hipLaunchKernelGGL((combine_kernel<N, 1>), grid, block, 0, s, y, y_rows, H, slot, w, \
                           K, out);                                                              \
        break;
    if (many) {
        if (rs.ppt == 1)
            hipLaunchKernelGGL((combine_kernel<1, 4>), grid, block, 0, s, y, y_rows, H, slot,
                               w, K, out);
        else
            hipLaunchKernelGGL((combine_kernel<2, 4>), grid, block, 0, s, y, y_rows, H, slot,
                               w, K, out);
        return hipGetLastError();
    }
    EP_PPT_SWITCH(rs.ppt, EP_COMBINE_CASE)
#undef EP_COMBINE_CASE
    return hipGetLastError();
}

hipError_t launch_combine_partial(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                                  const float *w, int S, int K, float *partial, hipStream_t s)
{
    if (S == 0)
        return hipSuccess;
    // The shapes of the bf16 combine in units of 4 channels (the same bytes
    // per thread): few rows with K < 12 take 8 slots per round, many source
    // slots (K >= 12) or few rows 4, otherwise 2 (a received row has few
    // valid slots: at prefill with 8 ranks, 1.4 on average).
    const bool many = K >= 12 || S < 1024;
    const bool few = S < 1024 && K < 12;
    RowShape rs = row_shape(H / 4, few ? 2 : (many ? 4 : 16));
    if ((uint64_t)S * rs.bd > 0xFFFFFFFFull)
        return hipErrorInvalidConfiguration;
    dim3 grid(S, rs.nseg), block(rs.bd);
#define EP_PARTIAL_LAUNCH(N, G_)                                                                \
    hipLaunchKernelGGL((partial_kernel<N, G_>), grid, block, 0, s, y, y_rows, H, slot, w, K,    \
                       partial)
    if (few) {
        if (rs.ppt == 1)
            EP_PARTIAL_LAUNCH(1, 8);
        else
            EP_PARTIAL_LAUNCH(2, 8);
        return hipGetLastError();
    }
    if (many) {
        switch (rs.ppt) {
        case 1: EP_PARTIAL_LAUNCH(1, 4); break;
        case 2: EP_PARTIAL_LAUNCH(2, 4); break;
        case 3: EP_PARTIAL_LAUNCH(3, 4); break;
        default: EP_PARTIAL_LAUNCH(4, 4); break;
        }
        return hipGetLastError();
    }
#define EP_PARTIAL_CASE(N) \
    case N:                \
        EP_PARTIAL_LAUNCH(N, 2); \
        break;
    switch (rs.ppt) {
        EP_PARTIAL_CASE(1)
        EP_PARTIAL_CASE(2)
        EP_PARTIAL_CASE(3)
        EP_PARTIAL_CASE(4)
        EP_PARTIAL_CASE(5)
        EP_PARTIAL_CASE(6)
        EP_PARTIAL_CASE(7)
        EP_PARTIAL_CASE(8)
        EP_PARTIAL_CASE(9)
        EP_PARTIAL_CASE(10)
        EP_PARTIAL_CASE(11)
        EP_PARTIAL_CASE(12)
        EP_PARTIAL_CASE(13)
        EP_PARTIAL_CASE(14)
        EP_PARTIAL_CASE(15)
        EP_PARTIAL_CASE(16)
    default:
        return hipErrorInvalidValue;
    }
#undef EP_PARTIAL_CASE
#undef EP_PARTIAL_LAUNCH
    return hipGetLastError();
}

hipError_t launch_ec_combine(const uint16_t *y, const float *w, int E, int C, int H,
                             const int32_t *tok_off, const int32_t *tok_ent, int T,
                             uint16_t *out, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    // At most 2 pieces per thread (so a popular token's row is spread over
    // more blocks) and 16 row pieces in flight per thread.
    RowShape rs = row_shape(H / 8, 2);
    if ((uint64_t)T * rs.bd > 0xFFFFFFFFull)
        return hipErrorInvalidConfiguration;
    dim3 grid(T, rs.nseg), block(rs.bd);
    if (rs.ppt == 1)
        hipLaunchKernelGGL((ec_combine_kernel<1, 16>), grid, block, 0, s, y, w, E * C, H, tok_off,
                           tok_ent, out);
    else
        hipLaunchKernelGGL((ec_combine_kernel<2, 8>), grid, block, 0, s, y, w, E * C, H, tok_off,
                           tok_ent, out);
    return hipGetLastError();
}

}  // namespace ep
