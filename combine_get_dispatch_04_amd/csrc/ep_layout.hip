// ep_layout.hip -- dispatch layout and stable slot ranks ("DeepEP-Ascend"
// README, API Overview: get_dispatch_layout; Environment Variables: the
// per-expert count and prefix-sum forms, and -1 meaning "not dispatched").
//
// topk_idx [T, K] is cut into chunks of CT whole tokens.  One block per
// chunk; each of its waves takes a contiguous run of the chunk's entries in
// row-major (t, k) order and walks it 64 entries at a time, keeping a
// running per-expert count in LDS.  Inside a 64-entry tile the entries with
// the same expert are found with one ballot per expert-id bit, so an
// entry's rank is (running count) + (same-expert lanes below it): a stable
// counting sort with no atomics.  The block then turns the per-wave counts
// into per-wave bases and adds them, leaving in `local_rank` each entry's
// rank among the chunk's entries of its expert, and writes the chunk's
// histogram.  The scan kernel turns the chunk histograms into per-chunk
// bases (column prefix over chunks) and the per-expert totals into counts
// and offsets.  ep_dispatch later places entry (t,k) of expert e at
// offsets[e] + chunk_base[t / CT][e] + local_rank[t, k].
#include "ep_common.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kEntriesPerLane = 8;   // target entries per lane and chunk
constexpr int kMaxWaves = 16;
constexpr int kLdsInts = 16384;      // 64 KiB per block
constexpr int kMaxRanks = 1024;

// Offsets from per-expert totals held in shared memory: an exclusive scan
// over E by the whole block.  Each thread owns a run of consecutive experts.
__device__ void offsets_from_totals(const int32_t *tot, int E, int32_t *offsets, int *tmp)
{
    int per = (E + blockDim.x - 1) / blockDim.x;
    int b0 = min(E, (int)threadIdx.x * per), b1 = min(E, b0 + per);
    int sum = 0;
    for (int e = b0; e < b1; ++e)
        sum += tot[e];
    int total;
    int ex = block_exclusive_scan(sum, tmp, &total);
    for (int e = b0; e < b1; ++e) {
        offsets[e] = ex;
        ex += tot[e];
    }
    if (threadIdx.x == 0)
        offsets[E] = total;
}

__global__ void __launch_bounds__(1024)
layout_chunk_kernel(const int32_t *__restrict__ topk_idx, int T, int K, int E, int R, int CT,
                    int nbits, int32_t *__restrict__ chunk_hist, int32_t *__restrict__ local_rank,
                    int32_t *__restrict__ rank_part, int32_t *__restrict__ inval_part,
                    uint8_t *__restrict__ is_token_in_rank, int32_t *__restrict__ counts,
                    int32_t *__restrict__ offsets, int32_t *__restrict__ tokens_per_rank,
                    int32_t *__restrict__ num_invalid)
{
    extern __shared__ int32_t lds[];
    const int waves = blockDim.x / kWave;
    int32_t *whist = lds;                 // [waves][E] running counts, then per-wave bases
    int32_t *tot = whist + waves * E;     // [E] chunk totals
    int32_t *rcnt = tot + E;              // [R] tokens per rank in this chunk
    int32_t *tmp = rcnt + R;              // [32] scratch
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int chunk = blockIdx.x;
    const bool single = gridDim.x == 1;
    const int t0 = chunk * CT;
    const int t1 = min(T, t0 + CT);
    const int64_t base = (int64_t)t0 * K;
    const int n = (t1 - t0) * K;

    for (int i = tid; i < waves * E; i += blockDim.x)
        whist[i] = 0;
    for (int i = tid; i < R; i += blockDim.x)
        rcnt[i] = 0;
    if (tid < 32)
        tmp[tid] = 0;
    __syncthreads();

    // ---- pass 1: per-wave stable ranks
    const int span = (((n + waves - 1) / waves) + kWave - 1) & ~(kWave - 1);
    const int lo = min(n, w * span), hi = min(n, lo + span);
    int32_t *myh = whist + w * E;
    int inval = 0;
    for (int s0 = lo; s0 < hi; s0 += kWave) {
        const int i = s0 + lane;
        const bool in = i < hi;
        const int e = in ? topk_idx[base + i] : -1;
        const bool ok = in && (unsigned)e < (unsigned)E;
        inval += (in && e != -1 && !ok) ? 1 : 0;
        const uint64_t peers = match_key(e, ok, nbits);
        if (ok) {
            const int r0 = myh[e];
            const int below = __popcll(peers & lanemask_lt(lane));
            if ((peers >> lane) == 1ull)         // highest lane of the group
                myh[e] = r0 + __popcll(peers);
            local_rank[base + i] = r0 + below;
        }
    }
    __syncthreads();

    // ---- per-wave bases (prefix over waves) and chunk totals
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int ww = 0; ww < waves; ++ww) {
            int h = whist[ww * E + e];
            whist[ww * E + e] = run;
            run += h;
        }
        tot[e] = run;
        chunk_hist[(int64_t)chunk * E + e] = single ? 0 : run;
        if (single)
            counts[e] = run;
    }
    __syncthreads();

    // ---- pass 2: add the wave's base to its entries' ranks
    if (w > 0) {
        for (int s0 = lo; s0 < hi; s0 += kWave) {
            const int i = s0 + lane;
            if (i < hi) {
                const int e = topk_idx[base + i];
                if ((unsigned)e < (unsigned)E)
                    local_rank[base + i] += myh[e];
            }
        }
    }

    // ---- ranks: is_token_in_rank rows and per-chunk tokens_per_rank
    const int per_rank = E / R;
    for (int t = t0 + tid; t < t1; t += blockDim.x) {
        const int32_t *row = topk_idx + (int64_t)t * K;
        if (R <= 64) {
            uint64_t m = 0;
            for (int k = 0; k < K; ++k) {
                int e = row[k];
                if ((unsigned)e < (unsigned)E)
                    m |= 1ull << (e / per_rank);
            }
            if (is_token_in_rank)
                for (int r = 0; r < R; ++r)
                    is_token_in_rank[(int64_t)t * R + r] = (uint8_t)((m >> r) & 1u);
            while (m) {
                int r = __ffsll((unsigned long long)m) - 1;
                atomicAdd(&rcnt[r], 1);
                m &= m - 1;
            }
        } else {
            if (is_token_in_rank)
                for (int r = 0; r < R; ++r)
                    is_token_in_rank[(int64_t)t * R + r] = 0;
            for (int k = 0; k < K; ++k) {
                int e = row[k];
                if ((unsigned)e >= (unsigned)E)
                    continue;
                int r = e / per_rank;
                bool first = true;
                for (int k2 = 0; k2 < k && first; ++k2) {
                    int e2 = row[k2];
                    if ((unsigned)e2 < (unsigned)E && e2 / per_rank == r)
                        first = false;
                }
                if (first) {
                    atomicAdd(&rcnt[r], 1);
                    if (is_token_in_rank)
                        is_token_in_rank[(int64_t)t * R + r] = 1;
                }
            }
        }
    }
    inval = wave_sum(inval);
    if (lane == 0 && inval)
        atomicAdd(&tmp[31], inval);
    __syncthreads();

    if (single) {
        if (tokens_per_rank)
            for (int r = tid; r < R; r += blockDim.x)
                tokens_per_rank[r] = rcnt[r];
        if (tid == 0)
            num_invalid[0] = tmp[31];
        __syncthreads();
        offsets_from_totals(tot, E, offsets, tmp);
    } else {
        for (int r = tid; r < R; r += blockDim.x)
            rank_part[(int64_t)chunk * R + r] = rcnt[r];
        if (tid == 0)
            inval_part[chunk] = tmp[31];
    }
}

// Column prefix over chunks: chunk_hist[c][e] becomes the number of entries
// of expert e in chunks before c; totals give counts and offsets.
__global__ void __launch_bounds__(1024)
layout_scan_kernel(int nchunk, int E, int R, int32_t *__restrict__ chunk_hist,
                   const int32_t *__restrict__ rank_part, const int32_t *__restrict__ inval_part,
                   int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                   int32_t *__restrict__ tokens_per_rank, int32_t *__restrict__ num_invalid)
{
    __shared__ int32_t tot[4096];
    __shared__ int tmp[32];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        int c = 0;
        for (; c + 8 <= nchunk; c += 8) {
            int h[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                h[u] = chunk_hist[(int64_t)(c + u) * E + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                chunk_hist[(int64_t)(c + u) * E + e] = run;
                run += h[u];
            }
        }
        for (; c < nchunk; ++c) {
            int h = chunk_hist[(int64_t)c * E + e];
            chunk_hist[(int64_t)c * E + e] = run;
            run += h;
        }
        tot[e] = run;
        counts[e] = run;
    }
    if (tokens_per_rank)
        for (int r = tid; r < R; r += blockDim.x) {
            int s = 0;
            for (int c = 0; c < nchunk; ++c)
                s += rank_part[(int64_t)c * R + r];
            tokens_per_rank[r] = s;
        }
    int inv = 0;
    for (int c = tid; c < nchunk; c += blockDim.x)
        inv += inval_part[c];
    int tot_inv;
    block_exclusive_scan(inv, tmp, &tot_inv);
    if (tid == 0)
        num_invalid[0] = tot_inv;
    __syncthreads();
    offsets_from_totals(tot, E, offsets, tmp);
}

}  // namespace

LayoutPlan make_layout_plan(int T, int K, int E, int R)
{
    LayoutPlan p{};
    p.T = T;
    p.K = K;
    p.E = E;
    p.R = R;
    p.nbits = 0;
    while ((1 << p.nbits) < E)
        ++p.nbits;
    // The chunking must not depend on R: ep_dispatch re-derives it from
    // (T, K, E) alone.  Shared memory is sized for the largest R.
    int fit = (kLdsInts - E - kMaxRanks - 32) / E;
    p.waves = fit < 1 ? 1 : (fit > kMaxWaves ? kMaxWaves : fit);
    long long target = (long long)p.waves * kWave * kEntriesPerLane;
    long long ct = target / K;
    if (ct < 1)
        ct = 1;
    if (ct > T && T > 0)
        ct = T;
    p.CT = (int)ct;
    p.nchunk = T > 0 ? (int)((T + ct - 1) / ct) : 0;
    // no more waves than 64-entry tiles in a chunk
    long long tiles = ((long long)p.CT * K + kWave - 1) / kWave;
    if (tiles < p.waves)
        p.waves = tiles < 1 ? 1 : (int)tiles;
    p.lds = (size_t)(p.waves * E + E + R + 32) * sizeof(int32_t);
    size_t off = 256;
    p.off_hist = off;
    off = align256(off + (size_t)p.nchunk * E * 4);
    p.off_rank = off;
    off = align256(off + (size_t)T * K * 4);
    p.off_rpart = off;
    off = align256(off + (size_t)p.nchunk * R * 4);
    p.off_ipart = off;
    off = align256(off + (size_t)p.nchunk * 4);
    p.bytes = off;
    return p;
}

hipError_t launch_layout(const LayoutPlan &p, const int32_t *topk_idx, int32_t *counts,
                         int32_t *offsets, int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                         int32_t *num_invalid, char *ws, hipStream_t s)
{
    int32_t *hist = reinterpret_cast<int32_t *>(ws + p.off_hist);
    int32_t *rank = reinterpret_cast<int32_t *>(ws + p.off_rank);
    int32_t *rpart = reinterpret_cast<int32_t *>(ws + p.off_rpart);
    int32_t *ipart = reinterpret_cast<int32_t *>(ws + p.off_ipart);
    if (p.nchunk > 0) {
        hipLaunchKernelGGL(layout_chunk_kernel, dim3(p.nchunk), dim3(p.waves * kWave), p.lds, s,
                           topk_idx, p.T, p.K, p.E, p.R, p.CT, p.nbits, hist, rank, rpart, ipart,
                           is_token_in_rank, counts, offsets, tokens_per_rank, num_invalid);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    if (p.nchunk != 1) {
        hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(1024), 0, s, p.nchunk, p.E, p.R, hist,
                           rpart, ipart, counts, offsets, tokens_per_rank, num_invalid);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace ep
