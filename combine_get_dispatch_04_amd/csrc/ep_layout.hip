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
// and offsets; when all of topk_idx fits one block (up to 16 waves x 64
// lanes x 8 entries), that block does this itself and there is one launch.
// ep_dispatch later places entry (t,k) of expert e at
// offsets[e] + chunk_base[t / CT][e] + local_rank[t, k].
//
// The sender pack of the expert-parallel exchange uses the same sort with
// ranks for keys ("rank keys"): entry (t,k) is keyed by the rank of its
// expert when it is the first of token t's valid entries on that rank, and
// is padding otherwise, so each key's entries are the tokens sent to that
// rank in token order, and the counts are the tokens per rank.
#include <algorithm>
#include <atomic>

#include "ep_common.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kMaxWaves = 16;
constexpr int kLdsInts = 16384;      // chunk kernel: 64 KiB of LDS per block
constexpr int kMaxRanks = 1024;
constexpr int kEpl = 8;              // entries per lane of a wave's run (at most)
constexpr int kSingleEpl = 4;        // at most this many tiles per wave in the one-block form
constexpr long long kTargetChunks = 64;
constexpr int kScanSeg = 256;        // chunks per column segment in the scan
// The scan's smallest tile: what 64 KiB holds next to E = 4096 totals and
// the 32-int scratch; the launch grows it to every column when the device's
// LDS allows.
constexpr int kScanTileInts = 16384 - 4096 - 32;

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

// One block per chunk of CT tokens (n = CT*K entries <= waves*64*epl), or,
// when one token's row is longer than that (CE > 0), per chunk of CE
// entries, so that a row may span chunks.  The chunk's entries are staged
// in shared memory; wave w walks entries [w*64*epl, (w+1)*64*epl) 64 at a
// time.  Expert ranks depend only on the row-major order of the entries, so
// they come out the same either way; the per-token work (rank marks, rank
// keys) reads a row's entries outside the chunk from global memory, and a
// token's rank marks are counted by the chunk its row starts in.  The kernels are short-lived and
// each CU runs them from a cold instruction cache, so the loops are kept
// compact (not unrolled) and their state lives in shared memory.
template <bool ROUNDS>
__global__ void __launch_bounds__(1024)
layout_chunk_kernel(const int32_t *__restrict__ topk_idx, int T, int K, int E, int R, int CT,
                    int CE, int nbits, int epl, int key_experts, int key_div, int64_t rstride,
                    int32_t *__restrict__ chunk_hist,
                    int32_t *__restrict__ local_rank, int32_t *__restrict__ rank_part,
                    int32_t *__restrict__ inval_part, uint8_t *__restrict__ is_token_in_rank,
                    int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                    int32_t *__restrict__ tokens_per_rank, int32_t *__restrict__ num_invalid)
{
    extern __shared__ int32_t lds[];
    if constexpr (ROUNDS) {
        // rounds of T tokens side by side (grid.y): round y's entries, its
        // tables `rstride` ints further into the workspace, and its outputs
        const int64_t y = blockIdx.y;
        topk_idx += y * T * K;
        chunk_hist += y * rstride;
        local_rank += y * rstride;
        rank_part += y * rstride;
        inval_part += y * rstride;
        counts += y * E;
        offsets += y * (E + 1);
        num_invalid += y;
        if (tokens_per_rank)
            tokens_per_rank += y * R;
        if (is_token_in_rank)
            is_token_in_rank += y * T * R;
    }
    const int waves = blockDim.x / kWave;
    const int nchunk = gridDim.x;
    const int per_wave = kWave * epl;                  // a power of two
    const int wave_shift = 31 - __builtin_clz(per_wave);
    const int cap = waves * per_wave;
    int32_t *whist = lds;                 // [waves][E] running counts, then per-wave bases
    int32_t *tot = whist + waves * E;     // [E] chunk totals
    int32_t *rcnt = tot + E;              // [R] tokens per rank in this chunk
    int32_t *tmp = rcnt + R;              // [32] scratch
    int32_t *ent = tmp + 32;              // [cap] the chunk's entries
    int32_t *rkl = ent + cap;             // [cap] rank inside the owning wave's run
    const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
    const int chunk = blockIdx.x;
    const bool single = nchunk == 1;
    // the chunk's entries [base, base + n), and the tokens whose rows start
    // in it, [t0, t1)
    int64_t base;
    int n, t0, t1;
    if (CE > 0) {
        base = (int64_t)chunk * CE;
        n = (int)min((int64_t)CE, (int64_t)T * K - base);
        t0 = (int)((base + K - 1) / K);
        t1 = (int)min((int64_t)T, (base + n + K - 1) / K);
    } else {
        t0 = chunk * CT;
        t1 = min(T, t0 + CT);
        base = (int64_t)t0 * K;
        n = (t1 - t0) * K;
    }
    // entry g of topk_idx (row-major): staged when in the chunk
    auto entry_at = [&](int64_t g) -> int {
        const int64_t i = g - base;
        return (i >= 0 && i < n) ? ent[i] : topk_idx[g];
    };

    // ---- stage the entries: 8 loads in flight per thread
    for (int i0 = 0; i0 < n; i0 += blockDim.x * 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x + tid;
            v[u] = i < n ? topk_idx[base + i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * blockDim.x + tid;
            if (i < n)
                ent[i] = v[u];
        }
    }
    for (int i = tid; i < waves * E; i += blockDim.x)
        whist[i] = 0;
    for (int i = tid; i < R; i += blockDim.x)
        rcnt[i] = 0;
    if (tid < 32)
        tmp[tid] = 0;
    __syncthreads();

    // ---- rank keys: E here counts ranks; the entries hold experts in
    // [0, key_experts), key_div of them per rank.  An entry keeps its rank if
    // no earlier entry of its token has a valid expert on that rank, and
    // becomes padding (-1) otherwise; an invalid expert stays invalid (-2).
    if (key_div > 0) {
        for (int i = tid; i < n; i += blockDim.x) {
            const int64_t g = base + i;
            const int64_t row0 = g / K * K;
            const int k = (int)(g - row0);
            const int e = ent[i];
            int key = e == -1 ? -1 : -2;
            if ((unsigned)e < (unsigned)key_experts) {
                const int r = e / key_div;
                key = r;
                for (int k2 = 0; k2 < k; ++k2) {
                    const int e2 = entry_at(row0 + k2);
                    if ((unsigned)e2 < (unsigned)key_experts && e2 / key_div == r) {
                        key = -1;
                        break;
                    }
                }
            }
            rkl[i] = key;
        }
        __syncthreads();
        for (int i = tid; i < n; i += blockDim.x)
            ent[i] = rkl[i];
        __syncthreads();
    }

    // ---- stable ranks inside the wave's run: running count + same-expert lanes below
    int32_t *myh = whist + w * E;
    const int lo = w * per_wave, hi = min(n, lo + per_wave);
    int inval = 0;
#pragma unroll 1
    for (int s0 = lo; s0 < hi; s0 += kWave) {
        const int i = s0 + lane;
        const int e = i < hi ? ent[i] : -1;
        const bool ok = (unsigned)e < (unsigned)E;
        inval += (e != -1 && !ok) ? 1 : 0;
        const uint64_t peers = match_key(e, ok, nbits);
        if (ok) {
            const int r0 = myh[e];
            if ((peers >> lane) == 1ull)           // highest lane of the group publishes
                myh[e] = r0 + __popcll(peers);
            rkl[i] = r0 + lanes_below(peers);
        }
    }
    __syncthreads();

    // ---- per-wave bases (prefix over waves) and chunk totals
    for (int x = tid; x < E; x += blockDim.x) {
        int run = 0;
        for (int ww = 0; ww < waves; ++ww) {
            int h = whist[ww * E + x];
            whist[ww * E + x] = run;
            run += h;
        }
        tot[x] = run;
        chunk_hist[(int64_t)x * nchunk + chunk] = single ? 0 : run;
        if (single)
            counts[x] = run;
    }
    __syncthreads();
    for (int i = tid; i < n; i += blockDim.x) {
        const int e = ent[i];
        if ((unsigned)e < (unsigned)E)
            local_rank[base + i] = rkl[i] + whist[(i >> wave_shift) * E + e];
    }

    // ---- ranks: is_token_in_rank rows and this chunk's tokens_per_rank
    const int per_rank = E / R;
    const int ntok = t1 - t0;
    if (R <= 64) {
        for (int tb = 0; tb < ntok; tb += blockDim.x) {    // same trip count for every lane
            const int tl = tb + tid;
            uint64_t m = 0;
            if (tl < ntok) {
                const int64_t row0 = (int64_t)(t0 + tl) * K;
#pragma unroll 8
                for (int k = 0; k < K; ++k) {
                    const int ee = entry_at(row0 + k);
                    if ((unsigned)ee < (unsigned)E)
                        m |= 1ull << (R == 1 ? 0 : ee / per_rank);
                }
                if (is_token_in_rank)
                    for (int r = 0; r < R; ++r)
                        is_token_in_rank[(int64_t)(t0 + tl) * R + r] = (uint8_t)((m >> r) & 1u);
            }
            for (int r = 0; r < R; ++r) {
                const int c = __popcll(ballot((m >> r) & 1u));
                if (lane == 0 && c)
                    atomicAdd(&rcnt[r], c);
            }
        }
    } else {
        for (int tl = tid; tl < ntok; tl += blockDim.x) {
            const int64_t row0 = (int64_t)(t0 + tl) * K;
            if (is_token_in_rank)
                for (int r = 0; r < R; ++r)
                    is_token_in_rank[(int64_t)(t0 + tl) * R + r] = 0;
            for (int k = 0; k < K; ++k) {
                const int ee = entry_at(row0 + k);
                if ((unsigned)ee >= (unsigned)E)
                    continue;
                const int r = ee / per_rank;
                bool first = true;
                for (int k2 = 0; k2 < k && first; ++k2) {
                    const int e2 = entry_at(row0 + k2);
                    if ((unsigned)e2 < (unsigned)E && e2 / per_rank == r)
                        first = false;
                }
                if (first) {
                    atomicAdd(&rcnt[r], 1);
                    if (is_token_in_rank)
                        is_token_in_rank[(int64_t)(t0 + tl) * R + r] = 1;
                }
            }
        }
    }
    if (inval)                                     // rare: no wave reduction
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
            rank_part[(int64_t)r * nchunk + chunk] = rcnt[r];
        if (tid == 0)
            inval_part[chunk] = tmp[31];
    }
}

// Column prefix over chunks.  The chunk tables are column-major
// ([column][chunk]): columns 0..E-1 are the expert histograms (rewritten in
// place with their exclusive prefix over chunks, i.e. the chunk bases, and
// summed into counts), columns E..E+R-1 the per-rank token counts and the
// last the invalid-entry counts (only summed).  The tables are contiguous,
// so tiles of (columns x chunks) are copied into shared memory with
// coalesced loads, one thread scans one column of the tile sequentially
// (rows padded by one int against bank conflicts), and the expert columns
// are copied back coalesced.  Columns longer than a tile are done in
// segments with the running sum kept in the column's thread.
template <bool ROUNDS>
__global__ void __launch_bounds__(1024)
layout_scan_kernel(int nchunk, int E, int R, int tile_ints, int64_t rstride,
                   int32_t *__restrict__ chunk_hist, const int32_t *__restrict__ rank_part,
                   const int32_t *__restrict__ inval_part, int32_t *__restrict__ counts,
                   int32_t *__restrict__ offsets, int32_t *__restrict__ tokens_per_rank,
                   int32_t *__restrict__ num_invalid)
{
    extern __shared__ int32_t sm[];
    if constexpr (ROUNDS) {
        const int64_t y = blockIdx.x;                 // one block per round
        chunk_hist += y * rstride;
        rank_part += y * rstride;
        inval_part += y * rstride;
        counts += y * E;
        offsets += y * (E + 1);
        num_invalid += y;
        if (tokens_per_rank)
            tokens_per_rank += y * R;
    }
    const int tid = threadIdx.x, bd = blockDim.x;
    const int ncol = E + R + 1;
    // a segment of a column holds up to `seg` chunks, seg a power of two so
    // that an element index splits into (column, chunk) by shift and mask
    int sh = 0;
    while ((1 << sh) < nchunk && (1 << sh) < kScanSeg)
        ++sh;
    const int seg = 1 << sh;
    const int ld = seg + 1;                       // odd row stride: no bank conflicts
    int cpt = tile_ints / ld;                     // columns per tile
    cpt = cpt < 1 ? 1 : (cpt > bd ? bd : cpt);
    int32_t *tile = sm;
    int32_t *tot = sm + tile_ints;                // [E]
    int *tmp = tot + E;                           // [32]
    for (int col0 = 0; col0 < ncol; col0 += cpt) {
        const int nc = min(cpt, ncol - col0);
        const int cnt = nc << sh;
        int carry = 0;                            // running sum of column col0 + tid
        for (int s0 = 0; s0 < nchunk; s0 += seg) {
            const int sl = min(seg, nchunk - s0);
            for (int q0 = 0; q0 < cnt; q0 += 8 * bd) {
                int v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int q = q0 + u * bd + tid;
                    const int cl = q >> sh, c = q & (seg - 1), col = col0 + cl;
                    const int32_t *src = col < E       ? chunk_hist + (int64_t)col * nchunk
                                         : col < E + R ? rank_part + (int64_t)(col - E) * nchunk
                                                       : inval_part;
                    v[u] = (q < cnt && c < sl) ? src[s0 + c] : 0;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int q = q0 + u * bd + tid;
                    if (q < cnt)
                        tile[(q >> sh) * ld + (q & (seg - 1))] = v[u];
                }
            }
            __syncthreads();
            if (tid < nc) {
                int32_t *row = tile + tid * ld;
                for (int c0 = 0; c0 < sl; c0 += 8) {    // 8 shared-memory reads in flight
                    int h[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        h[u] = c0 + u < sl ? row[c0 + u] : 0;
#pragma unroll
                    for (int u = 0; u < 8; ++u)
                        if (c0 + u < sl) {
                            row[c0 + u] = carry;
                            carry += h[u];
                        }
                }
            }
            __syncthreads();
            for (int q = tid; q < cnt; q += bd) {
                const int cl = q >> sh, c = q & (seg - 1), col = col0 + cl;
                if (col < E && c < sl)
                    chunk_hist[(int64_t)col * nchunk + s0 + c] = tile[cl * ld + c];
            }
            __syncthreads();
        }
        if (tid < nc) {
            const int col = col0 + tid;
            if (col < E) {
                tot[col] = carry;
                counts[col] = carry;
            } else if (col < E + R) {
                if (tokens_per_rank)
                    tokens_per_rank[col - E] = carry;
            } else {
                num_invalid[0] = carry;
            }
        }
    }
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
    // (T, K, E) alone, so shared memory is sized for the largest R.  A wave
    // with `epl` entries per lane stages and ranks 64 * epl entries (two
    // ints each in shared memory, next to its E-entry histogram).
    auto wmax_for = [&](int epl) {
        int fit = (kLdsInts - E - kMaxRanks - 32) / (E + 2 * kWave * epl);
        return fit < 1 ? 1 : (fit > kMaxWaves ? kMaxWaves : fit);
    };
    // A wave's 64-entry tiles form a dependent chain (shared-memory count,
    // ballots, count update), measured at about 0.85 us per tile, so runs
    // are kept short and spread over many waves.  An input that one block
    // covers with at most kSingleEpl tiles per wave takes one block, which
    // also finishes the scan: one launch (8.3 us with 1 tile per wave, 10.2
    // with 4; with 8 it was 13.7 us against 11.7 for chunks and a scan).
    // Otherwise: the fewest entries per lane that keep about kTargetChunks
    // chunks (64 rather than 32: the large workload's layout 27.6 -> 24.9 us
    // with 4 tiles per wave instead of 8, and the same scan tile).
    const long long n = (long long)T * K;
    long long cap = 0;
    for (int epl = 1; epl <= kSingleEpl; epl *= 2) {
        const long long c = (long long)wmax_for(epl) * kWave * epl;
        if (n <= c) {
            p.epl = epl;
            cap = c;
            break;
        }
    }
    if (cap == 0) {
        p.epl = 1;
        while (p.epl < kEpl && n > kTargetChunks * wmax_for(p.epl) * kWave * p.epl)
            p.epl *= 2;
        cap = (long long)wmax_for(p.epl) * kWave * p.epl;
        while (cap < K && p.epl < kEpl) {   // a chunk holds one token if it can
            p.epl *= 2;
            cap = (long long)wmax_for(p.epl) * kWave * p.epl;
        }
    }
    const int wmax = wmax_for(p.epl);
    const long long per_wave = (long long)kWave * p.epl;
    if (cap < K) {
        // a row longer than a chunk: chunks of cap entries, rows spanning them
        p.CE = (int)cap;
        p.CT = 1;
        p.nchunk = (int)((n + cap - 1) / cap);
        p.waves = wmax;
    } else {
        long long ct = cap / K;
        if (ct < 1)
            ct = 1;
        if (ct > T && T > 0)
            ct = T;
        p.CT = (int)ct;
        p.CE = 0;
        p.nchunk = T > 0 ? (int)((T + ct - 1) / ct) : 0;
        long long wv = ((long long)p.CT * K + per_wave - 1) / per_wave;
        p.waves = wv < 1 ? 1 : (wv > wmax ? wmax : (int)wv);
    }
    p.lds = (size_t)(p.waves * E + E + R + 32 + 2 * p.waves * per_wave) * sizeof(int32_t);
    size_t off = 256;
    p.off_hist = off;
    off = align256(off + (size_t)p.nchunk * E * 4);
    p.off_rank = off;
    off = align256(off + (size_t)T * K * 4);
    p.off_rpart = off;
    off = align256(off + (size_t)p.nchunk * R * 4);
    p.off_ipart = off;
    off = align256(off + (size_t)p.nchunk * 4);
    p.off_tamax = off;
    off = align256(off + (size_t)T * 4);
    p.bytes = off;
    return p;
}

RankPlan make_rank_plan(int T, int K, int E, int R)
{
    RankPlan rp{};
    rp.lp = make_layout_plan(T, K, R, 1);
    rp.lp.key_experts = E;
    rp.lp.key_div = E / R;
    rp.off_misc = rp.lp.bytes;
    rp.bytes = align256(rp.off_misc + 4);
    return rp;
}

hipError_t launch_layout(const LayoutPlan &p, const int32_t *topk_idx, int32_t *counts,
                         int32_t *offsets, int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                         int32_t *num_invalid, char *ws, hipStream_t s, int rounds,
                         size_t round_bytes)
{
    int32_t *hist = reinterpret_cast<int32_t *>(ws + p.off_hist);
    int32_t *rank = reinterpret_cast<int32_t *>(ws + p.off_rank);
    int32_t *rpart = reinterpret_cast<int32_t *>(ws + p.off_rpart);
    int32_t *ipart = reinterpret_cast<int32_t *>(ws + p.off_ipart);
    const int64_t rstride = (int64_t)(round_bytes / sizeof(int32_t));
    if ((p.CE > 0 ? (long long)p.CE : (long long)p.CT * p.K) > (long long)p.waves * kWave * p.epl)
        return hipErrorInvalidValue;     // a chunk's entries must fit its waves
    if (rounds < 1 || rounds > 65535 || (rounds > 1 && round_bytes % 256 != 0))
        return hipErrorInvalidValue;
    // the single-call form gets kernels without the round offsets
    auto chunk_kernel = rounds > 1 ? layout_chunk_kernel<true> : layout_chunk_kernel<false>;
    auto scan_kernel = rounds > 1 ? layout_scan_kernel<true> : layout_scan_kernel<false>;
    if (p.nchunk > 0) {
        hipLaunchKernelGGL(chunk_kernel, dim3(p.nchunk, rounds), dim3(p.waves * kWave),
                           p.lds, s, topk_idx, p.T, p.K, p.E, p.R, p.CT, p.CE, p.nbits, p.epl,
                           p.key_experts, p.key_div, rstride, hist, rank, rpart, ipart,
                           is_token_in_rank, counts, offsets, tokens_per_rank, num_invalid);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    if (p.nchunk != 1) {
        // One tile holds every column when the device's LDS allows (gfx950:
        // 160 KiB per block); otherwise the columns go in several tiles.
        int seg = 1;
        while (seg < p.nchunk && seg < kScanSeg)
            seg <<= 1;
        const long long want = (long long)(p.E + p.R + 1) * (seg + 1);
        const long long room = (long long)lds_limit() / 4 - p.E - 32;
        const int tile = (int)std::max<long long>(kScanTileInts, std::min(want, room));
        const size_t dyn = (size_t)(tile + p.E + 32) * sizeof(int32_t);
        if (dyn > 65536) {
            hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(scan_kernel),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)dyn);
            if (err != hipSuccess)
                return err;
        }
        hipLaunchKernelGGL(scan_kernel, dim3(rounds), dim3(1024), dyn, s, p.nchunk, p.E,
                           p.R, tile, rstride, hist, rpart, ipart, counts, offsets,
                           tokens_per_rank, num_invalid);
        return hipGetLastError();
    }
    return hipSuccess;
}

int lds_limit()
{
    // per-device cache; callers on several host threads may race to fill
    // it, each with the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return 65536;
    }
    if (dev < 64) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess ||
        v <= 0) {
        (void)hipGetLastError();
        v = 65536;
    }
    if (dev < 64)
        cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

}  // namespace ep
