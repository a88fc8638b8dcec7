// ep_expert_choice.hip -- expert-choice dispatch ("[Feature Request] Support
// Expert-Choice Routing via Native Expert-Centric API ([num_experts,
// capacity])", Proposed Solutions, Solution 1).
//
// token_indices [E, C] lists, per expert, the tokens it picked.  Two results:
//   * the copy recv[j] = x[token_indices[j]] for flat entries j = e*C + c;
//   * the inverse map (token -> its entries j, ascending), which is the
//     handle that combine walks.
// The copy is entry-major: every block copies the same number of rows
// however unevenly the picks fall on tokens (in the expert-choice workload
// 27 tokens are picked by all 64 experts and 7198 by none).  A token's x row
// is read from HBM once; the other entries that picked it find it in L2 or
// the MALL.
//
// The inverse map is a stable counting sort of the entries by token.  When
// T * ceil(E/64) 64-bit words fit in one block's LDS, one block builds it:
// each token gets a bitmask of the experts that picked it (LDS atomic OR).
// A token's entries in ascending j are exactly its experts in ascending
// order, so an entry's rank inside its token is the number of mask bits
// below its expert and the token's count is the mask's popcount; no sort is
// needed.  If an OR finds its bit already set, some expert listed a token
// twice; the block then switches to counters, places the entries with
// atomics and orders each token's range by rank (the number of smaller
// entries in the range).
//
// The copy does not depend on the inverse map, so both run in one launch:
// block 0 builds the map while the other blocks copy rows.  All blocks then
// have 1024 threads and the masks' LDS, which is kept to half a CU's LDS so
// that two blocks (32 waves) still fit on every CU.  With larger masks the
// map gets a launch of its own before the copy; when they do not fit at all,
// five launches do the same steps with the counters in the workspace.
#include "ep_common.h"
#include "ep_internal.h"

#include <initializer_list>

namespace ep {

namespace {

constexpr int kInvThreads = 1024;
constexpr int kInvEnt = 8;              // entries per thread per pass
constexpr int kScanPer = 8;             // tokens per lane per scan pass
constexpr size_t kFusedLds = 81920 - 256;   // two blocks per CU of 160 KiB

// e = j / C for 0 <= j < E*C < 2^31.  The one-block map only runs when
// T*ceil(E/64) 64-bit words fit in LDS, so E < 2^21; the fp32 estimate then
// errs by less than one and the two integer checks correct it (no product
// exceeds E*C).
__device__ __forceinline__ int expert_of(int j, int C, float inv_c)
{
    int e = (int)((float)j * inv_c);
    if (e * C > j)
        --e;
    else if ((e + 1) * C <= j)
        ++e;
    return e;
}

__device__ __forceinline__ int mask_count(const uint64_t *m, int W)
{
    int c = 0;
    for (int w = 0; w < W; ++w)
        c += __popcll(m[w]);
    return c;
}

// Bits of m below bit e (experts before e that picked the token); with W1
// the mask is one word (e < 64).
template <bool W1 = false>
__device__ __forceinline__ int mask_rank(const uint64_t *m, int e)
{
    if (W1)
        return __popcll(m[0] & ((1ull << (e & 63)) - 1ull));
    int c = 0;
    const int w1 = e >> 6;
    for (int w = 0; w < w1; ++w)
        c += __popcll(m[w]);
    return c + __popcll(m[w1] & ((1ull << (e & 63)) - 1ull));
}

// Exclusive scan of per-token counts cnt_of(t) into tok_off[0..T]; with
// `cursor` the offsets also go there.  A pass covers blockDim.x * kScanPer
// tokens: wave w takes 64*kScanPer consecutive tokens, lane l the tokens
// l, l+64, ... of them, so every load and store of a wave is contiguous.
// `tmp` holds >= 17 ints of LDS.  Returns the total (in every thread).
template <typename F>
__device__ __forceinline__ int scan_tokens(int T, F cnt_of, int32_t *__restrict__ tok_off,
                                           int32_t *cursor, int *tmp)
{
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nw = blockDim.x / kWave;
    int carry = 0;
    for (int64_t t0 = 0; t0 < T; t0 += (int64_t)blockDim.x * kScanPer) {
        const int64_t base = t0 + (int64_t)wave * (kWave * kScanPer) + lane;
        int c[kScanPer], ex[kScanPer];
        int run = 0;
#pragma unroll
        for (int u = 0; u < kScanPer; ++u) {
            const int64_t t = base + u * kWave;
            c[u] = t < T ? cnt_of((int)t) : 0;
        }
#pragma unroll
        for (int u = 0; u < kScanPer; ++u) {
            const int inc = wave_inclusive_scan(c[u], lane);
            ex[u] = run + inc - c[u];
            run += __builtin_amdgcn_readlane(inc, kWave - 1);
        }
        if (lane == 0)
            tmp[wave] = run;
        __syncthreads();
        if (wave == 0) {
            const int s = lane < nw ? tmp[lane] : 0;
            const int si = wave_inclusive_scan(s, lane);
            if (lane < nw)
                tmp[lane] = si - s;
            if (lane == kWave - 1)
                tmp[16] = si;
        }
        __syncthreads();
        const int wbase = carry + tmp[wave];
        carry += tmp[16];
#pragma unroll
        for (int u = 0; u < kScanPer; ++u) {
            const int64_t t = base + u * kWave;
            if (t < T) {
                tok_off[t] = wbase + ex[u];
                if (cursor)
                    cursor[t] = wbase + ex[u];
            }
        }
        __syncthreads();                    // tmp is reused by the next pass
    }
    if (tid == 0)
        tok_off[T] = carry;
    return carry;
}

// Token t's entries are tmp[b .. b+m) in any order; write them ascending.
__device__ __forceinline__ void rank_place(const int32_t *tmp, int b, int m, int val,
                                           int32_t *__restrict__ tok_ent)
{
    int rank = 0;
    for (int q = 0; q < m; ++q)
        rank += tmp[b + q] < val ? 1 : 0;
    tok_ent[b + rank] = val;
}

// Some expert lists a token more than once: count, place, then order.  The
// mask words (>= (T+1)*4 bytes of LDS) hold counters, then cursors.
__device__ __forceinline__ void invert_with_duplicates(const int32_t *__restrict__ ti, int T,
                                                       int n, int32_t *__restrict__ tok_off,
                                                       int32_t *__restrict__ tok_ent,
                                                       int32_t *__restrict__ tmp_ent,
                                                       uint64_t *masks, int *red)
{
    const int tid = threadIdx.x, bd = blockDim.x;
    __syncthreads();
    int32_t *cur = reinterpret_cast<int32_t *>(masks);
    for (int i = tid; i <= T; i += bd)
        cur[i] = 0;
    __syncthreads();
    for (int64_t j = tid; j < n; j += bd) {
        const int v = ti[j];
        if ((unsigned)v < (unsigned)T)
            atomicAdd(&cur[v], 1);
    }
    __syncthreads();
    const int total = scan_tokens(T, [&](int t) { return cur[t]; }, tok_off, cur, red);
    __syncthreads();
    for (int64_t j = tid; j < n; j += bd) {
        const int v = ti[j];
        if ((unsigned)v < (unsigned)T)
            tmp_ent[atomicAdd(&cur[v], 1)] = (int32_t)j;
    }
    __threadfence();
    __syncthreads();
    for (int64_t p = tid; p < total; p += bd) {
        const int val = tmp_ent[p];
        const int t = ti[val];
        const int b = tok_off[t];
        rank_place(tmp_ent, b, tok_off[t + 1] - b, val, tok_ent);
    }
}

// The inverse map when every thread holds all of its entries in registers
// (n <= blockDim.x * kInvRes): thread i owns entries [kInvRes*i, kInvRes*i +
// kInvRes), loaded once with 16-byte buffer loads; its expert index starts
// from one division and steps along.  The ORs return nothing: without
// duplicates every valid entry sets a bit of its own, so the masks'
// popcount total equals the number of valid entries, and a smaller total
// means some expert listed a token twice.  Ranks are taken from the masks
// first; the scan then writes the offsets over the mask words (offset t sits
// in bytes [4t, 4t+4), below the words of every token a later scan pass
// still reads).
constexpr int kInvRes = 16;

// W1: one mask word per token (E <= 64), known at compile time.
template <bool W1>
__device__ __forceinline__ void invert_resident(const int32_t *__restrict__ ti, int T, int C,
                                                int Wr, int n, float inv_c,
                                                int32_t *__restrict__ tok_off,
                                                int32_t *__restrict__ tok_ent,
                                                int32_t *__restrict__ num_invalid,
                                                int32_t *__restrict__ tmp_ent, uint64_t *masks,
                                                int *red)
{
    const int tid = threadIdx.x;
    const int W = W1 ? 1 : Wr;
    const int jb = tid * kInvRes;
    int v[kInvRes];
    {
        const rsrc_t src = row_rsrc(ti, n * 4);        // reads past n return 0
#pragma unroll
        for (int q = 0; q < kInvRes / 4; ++q) {
            const u32x4 w = row_ld16_cached(src, (jb + 4 * q) * 4);
            v[4 * q] = (int)w.x;
            v[4 * q + 1] = (int)w.y;
            v[4 * q + 2] = (int)w.z;
            v[4 * q + 3] = (int)w.w;
        }
        if (jb + kInvRes > n) {
#pragma unroll
            for (int u = 0; u < kInvRes; ++u)
                if (jb + u >= n)
                    v[u] = -1;
        }
    }
    const int e0 = jb < n ? expert_of(jb, C, inv_c) : 0;
    const int c0 = jb - e0 * C;
    int inval = 0, valid = 0;
    {
        int e = e0, c = c0;
#pragma unroll
        for (int u = 0; u < kInvRes; ++u) {
            if ((unsigned)v[u] < (unsigned)T) {
                __hip_atomic_fetch_or(&masks[(int64_t)v[u] * W + (e >> 6)], 1ull << (e & 63),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                ++valid;
            } else if (v[u] != -1) {
                ++inval;
            }
            if (++c == C) {
                c = 0;
                ++e;
            }
        }
    }
    if (inval)
        atomicAdd(&red[31], inval);
    if (valid)
        atomicAdd(&red[30], valid);
    __syncthreads();
    if (tid == 0)
        num_invalid[0] = red[31];
    const int n_valid = red[30];

    // token | rank << 17, or -1: the rank is below n <= 2^14 and the token
    // below 2^17 (T * 8 bytes fit in LDS)
    {
        int e = e0, c = c0;
#pragma unroll
        for (int u = 0; u < kInvRes; ++u) {
            if ((unsigned)v[u] < (unsigned)T)
                v[u] |= mask_rank<W1>(masks + (int64_t)v[u] * W, e) << 17;
            else
                v[u] = -1;
            if (++c == C) {
                c = 0;
                ++e;
            }
        }
    }
    int32_t *off = reinterpret_cast<int32_t *>(masks);
    const int total = scan_tokens(T, [&](int t) { return mask_count(masks + (int64_t)t * W, W); },
                                  tok_off, off, red);
    if (total != n_valid) {
        invert_with_duplicates(ti, T, n, tok_off, tok_ent, tmp_ent, masks, red);
        return;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kInvRes; ++u)
        if (v[u] >= 0)
            tok_ent[off[v[u] & 0x1FFFF] + (v[u] >> 17)] = jb + u;
}

__device__ __forceinline__ void clear_masks(uint64_t *masks, int64_t nwords, int *red)
{
    for (int64_t i = threadIdx.x; i < nwords; i += blockDim.x)
        masks[i] = 0ull;
    if (threadIdx.x < 32)
        red[threadIdx.x] = 0;
    __syncthreads();
}

__device__ __forceinline__ void invert_block(const int32_t *__restrict__ ti, int T, int C, int W, int n,
                             float inv_c, int32_t *__restrict__ tok_off,
                             int32_t *__restrict__ tok_ent, int32_t *__restrict__ num_invalid,
                             int32_t *__restrict__ tmp_ent, uint64_t *masks, int *red)
{
    const int tid = threadIdx.x, bd = blockDim.x;
    clear_masks(masks, (int64_t)T * W, red);
    if ((int64_t)n <= (int64_t)bd * kInvRes) {
        if (W == 1)
            invert_resident<true>(ti, T, C, W, n, inv_c, tok_off, tok_ent, num_invalid, tmp_ent,
                                  masks, red);
        else
            invert_resident<false>(ti, T, C, W, n, inv_c, tok_off, tok_ent, num_invalid, tmp_ent,
                                   masks, red);
        return;
    }

    int inval = 0;
    bool dup = false;
    for (int64_t j0 = 0; j0 < n; j0 += (int64_t)bd * kInvEnt) {
        int v[kInvEnt];
#pragma unroll
        for (int u = 0; u < kInvEnt; ++u) {
            const int64_t j = j0 + u * bd + tid;
            v[u] = j < n ? ti[j] : -1;
        }
#pragma unroll
        for (int u = 0; u < kInvEnt; ++u) {
            const int j = (int)(j0 + u * bd + tid);
            if ((unsigned)v[u] < (unsigned)T) {
                const int e = expert_of(j, C, inv_c);
                const unsigned long long bit = 1ull << (e & 63);
                const unsigned long long old = atomicOr(
                    reinterpret_cast<unsigned long long *>(&masks[(int64_t)v[u] * W + (e >> 6)]),
                    bit);
                dup |= (old & bit) != 0ull;
            } else if (v[u] != -1) {
                ++inval;
            }
        }
    }
    if (inval)
        atomicAdd(&red[31], inval);
    const bool any_dup = __syncthreads_or(dup) != 0;
    if (tid == 0)
        num_invalid[0] = red[31];

    if (!any_dup) {
        scan_tokens(T, [&](int t) { return mask_count(masks + (int64_t)t * W, W); }, tok_off,
                    nullptr, red);
        __threadfence();                    // tok_off is read back from L2 below
        __syncthreads();
        for (int64_t j0 = 0; j0 < n; j0 += (int64_t)bd * kInvEnt) {
            int v[kInvEnt], r[kInvEnt], base[kInvEnt];
#pragma unroll
            for (int u = 0; u < kInvEnt; ++u) {
                const int64_t j = j0 + u * bd + tid;
                v[u] = j < n ? ti[j] : -1;
            }
#pragma unroll
            for (int u = 0; u < kInvEnt; ++u) {
                const bool ok = (unsigned)v[u] < (unsigned)T;
                const int j = (int)(j0 + u * bd + tid);
                r[u] = ok ? mask_rank(masks + (int64_t)v[u] * W, expert_of(j, C, inv_c)) : 0;
                base[u] = ok ? tok_off[v[u]] : 0;
            }
#pragma unroll
            for (int u = 0; u < kInvEnt; ++u)
                if ((unsigned)v[u] < (unsigned)T)
                    tok_ent[base[u] + r[u]] = (int)(j0 + u * bd + tid);
        }
        return;
    }

    invert_with_duplicates(ti, T, n, tok_off, tok_ent, tmp_ent, masks, red);
}

__global__ void __launch_bounds__(kInvThreads)
ec_invert_kernel(const int32_t *__restrict__ ti, int T, int C, int W, int n, float inv_c,
                 int32_t *__restrict__ tok_off, int32_t *__restrict__ tok_ent,
                 int32_t *__restrict__ num_invalid, int32_t *__restrict__ tmp_ent)
{
    extern __shared__ uint64_t masks[];
    __shared__ int red[32];
    invert_block(ti, T, C, W, n, inv_c, tok_off, tok_ent, num_invalid, tmp_ent, masks, red);
}

// recv[j] = x[t] for one row segment: PPT pieces per thread, `bdr` threads,
// thread lt.  The x row is loaded with the default cache policy: other
// entries that picked the same token read it again.
template <int PPT>
__device__ __forceinline__ void copy_row(const uint16_t *__restrict__ x, int H, int t, int j,
                                         int seg0, int lt, int bdr, uint16_t *__restrict__ recv)
{
    const int pieces = H >> 3;
    const rsrc_t src = row_rsrc(x + (size_t)t * H, pieces * 16);
    const rsrc_t dst = row_rsrc(recv + (size_t)j * H, pieces * 16);
    u32x4 v[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k)
        v[k] = row_ld16_cached(src, (seg0 + lt + k * bdr) * 16);
#pragma unroll
    for (int k = 0; k < PPT; ++k)
        row_st16(dst, (seg0 + lt + k * bdr) * 16, v[k]);
}

// Block 0 builds the inverse map (E <= 64, n <= 1024 * kInvRes); block b >= 1 copies entries
// (b-1)*spb .. (b-1)*spb + spb-1, one per group of bdr = 1024/spb threads
// (a whole number of waves, so the entry is wave-uniform).
template <int PPT>
__global__ void __launch_bounds__(kInvThreads, 8)     // 8 waves per SIMD: two blocks per CU
ec_dispatch_fused_kernel(const uint16_t *__restrict__ x, int H, const int32_t *__restrict__ ti,
                         int T, int C, int W, int n, float inv_c, int spb,
                         uint16_t *__restrict__ recv, int32_t *__restrict__ tok_off,
                         int32_t *__restrict__ tok_ent, int32_t *__restrict__ num_invalid,
                         int32_t *__restrict__ tmp_ent)
{
    extern __shared__ uint64_t masks[];
    __shared__ int red[32];
    if (blockIdx.x == 0) {
        if (blockIdx.y == 0) {
            clear_masks(masks, T, red);
            invert_resident<true>(ti, T, C, 1, n, inv_c, tok_off, tok_ent, num_invalid, tmp_ent,
                                  masks, red);
        }
        return;
    }
    const int bdr = blockDim.x / spb;
    const int sub = threadIdx.x / bdr, lt = threadIdx.x % bdr;
    const int64_t j = (int64_t)(blockIdx.x - 1) * spb + sub;
    if (j >= n)
        return;
    const int t = __builtin_amdgcn_readfirstlane(ti[j]);
    if ((unsigned)t >= (unsigned)T)
        return;
    copy_row<PPT>(x, H, t, (int)j, blockIdx.y * PPT * bdr, lt, bdr, recv);
}

// ------------------------------------------------ multi-launch inverse map
__global__ void fill_kernel(int32_t *__restrict__ p, int64_t n, int32_t v)
{
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void ec_count_kernel(const int32_t *__restrict__ ti, int64_t n, int T,
                                int32_t *__restrict__ cnt, int32_t *__restrict__ ninv)
{
    int inval = 0;
    for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n;
         j += (int64_t)gridDim.x * blockDim.x) {
        int v = ti[j];
        if ((unsigned)v < (unsigned)T)
            atomicAdd(&cnt[v], 1);
        else if (v != -1)
            ++inval;
    }
    inval = wave_sum(inval);
    if ((threadIdx.x % kWave) == 0 && inval)
        atomicAdd(ninv, inval);
}

__global__ void __launch_bounds__(kInvThreads)
ec_scan_kernel(const int32_t *__restrict__ cnt, int T, int32_t *__restrict__ tok_off,
               int32_t *__restrict__ cursor, const int32_t *__restrict__ ninv_ws,
               int32_t *__restrict__ num_invalid)
{
    __shared__ int tmp[32];
    scan_tokens(T, [&](int t) { return cnt[t]; }, tok_off, cursor, tmp);
    if (threadIdx.x == 0)
        num_invalid[0] = ninv_ws[0];
}

__global__ void ec_place_kernel(const int32_t *__restrict__ ti, int64_t n, int T,
                                int32_t *__restrict__ cursor, int32_t *__restrict__ tmp)
{
    for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < n;
         j += (int64_t)gridDim.x * blockDim.x) {
        int v = ti[j];
        if ((unsigned)v < (unsigned)T) {
            int pos = atomicAdd(&cursor[v], 1);
            tmp[pos] = (int32_t)j;
        }
    }
}

// One block per token: order its range, staging it through LDS in tiles.
constexpr int kSortTile = 1024;

__global__ void __launch_bounds__(256)
ec_sort_kernel(const int32_t *__restrict__ tok_off, const int32_t *__restrict__ tmp,
               int32_t *__restrict__ tok_ent)
{
    __shared__ int32_t tile[kSortTile];
    const int t = blockIdx.x;
    const int b = tok_off[t], n = tok_off[t + 1] - b;
    const int tid = threadIdx.x, bd = blockDim.x;
    if (n <= 1) {
        if (n == 1 && tid == 0)
            tok_ent[b] = tmp[b];
        return;
    }
    for (int a0 = 0; a0 < n; a0 += bd) {
        const int a = a0 + tid;
        const int val = a < n ? tmp[b + a] : 0x7FFFFFFF;
        int rank = 0;
        for (int m0 = 0; m0 < n; m0 += kSortTile) {
            const int m1 = min(n, m0 + kSortTile);
            __syncthreads();
            for (int m = m0 + tid; m < m1; m += bd)
                tile[m - m0] = tmp[b + m];
            __syncthreads();
            for (int m = 0; m < m1 - m0; ++m)
                rank += tile[m] < val ? 1 : 0;
        }
        if (a < n)
            tok_ent[b + rank] = val;
    }
}

// One block (bdr threads) per (entry, row segment).
template <int PPT>
__global__ void __launch_bounds__(256)
ec_copy_kernel(const uint16_t *__restrict__ x, int H, const int32_t *__restrict__ ti, int T,
               uint16_t *__restrict__ recv)
{
    const int j = blockIdx.x;
    const int t = ti[j];
    if ((unsigned)t >= (unsigned)T)
        return;
    copy_row<PPT>(x, H, t, j, blockIdx.y * PPT * blockDim.x, threadIdx.x, blockDim.x, recv);
}

struct RowShape {
    int bd, ppt, nseg;
};

// Fewest idle lanes over the given thread counts with at most `maxppt`
// pieces per thread; more row segments (grid.y) when a row is longer.
RowShape row_shape(int pieces, int maxppt, std::initializer_list<int> bds)
{
    RowShape best{64, 1, 1};
    long long best_waste = -1;
    for (int bd : bds) {
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

int grid_for(int64_t n, int bd)
{
    int64_t g = (n + bd - 1) / bd;
    if (g < 1)
        g = 1;
    if (g > 4096)
        g = 4096;
    return (int)g;
}

#define EP_EC_PPT_SWITCH(PPT_VAR, CASE) \
    switch (PPT_VAR) {                  \
        CASE(1)                         \
        CASE(2)                         \
        CASE(3)                         \
        CASE(4)                         \
        CASE(5)                         \
        CASE(6)                         \
        CASE(7)                         \
        CASE(8)                         \
    default:                            \
        return hipErrorInvalidValue;    \
    }

hipError_t launch_copy(const uint16_t *x, int H, const int32_t *ti, int T, int64_t n,
                       uint16_t *recv, hipStream_t s)
{
    RowShape rs = row_shape(H / 8, 8, {256, 128, 64});
    if ((uint64_t)n * rs.bd > 0xFFFFFFFFull)    // work-items per grid dimension fit in 32 bits
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)n, rs.nseg), block(rs.bd);
#define EP_EC_COPY_CASE(N)                                                                      \
    case N:                                                                                     \
        hipLaunchKernelGGL((ec_copy_kernel<N>), grid, block, 0, s, x, H, ti, T, recv);        \
        break;
    EP_EC_PPT_SWITCH(rs.ppt, EP_EC_COPY_CASE)
#undef EP_EC_COPY_CASE
    return hipGetLastError();
}

hipError_t launch_fused(const uint16_t *x, int H, const int32_t *ti, int T, int C, int W,
                        int64_t n, size_t dyn, uint16_t *recv, int32_t *tok_off,
                        int32_t *tok_ent, int32_t *num_invalid, int32_t *tmp, hipStream_t s)
{
    RowShape rs = row_shape(H / 8, 8, {256, 128, 64, 512, 1024});
    const int spb = kInvThreads / rs.bd;
    const int64_t nblk = 1 + (n + spb - 1) / spb;
    if (nblk * kInvThreads > 0xFFFFFFFFll)
        return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)nblk, rs.nseg), block(kInvThreads);
    const float inv_c = 1.0f / (float)C;
#define EP_EC_FUSED_CASE(N)                                                                     \
    case N:                                                                                     \
        hipLaunchKernelGGL((ec_dispatch_fused_kernel<N>), grid, block, dyn, s, x, H, ti, T, C, \
                           W, (int)n, inv_c, spb, recv, tok_off, tok_ent, num_invalid, tmp);  \
        break;
    EP_EC_PPT_SWITCH(rs.ppt, EP_EC_FUSED_CASE)
#undef EP_EC_FUSED_CASE
    return hipGetLastError();
}

}  // namespace

EcPlan make_ec_plan(int T, int E, int C)
{
    EcPlan p{};
    p.T = T;
    p.E = E;
    p.C = C;
    size_t off = 256;
    p.off_misc = off;                       // [0] invalid counter
    off = align256(off + 64);
    p.off_cnt = off;
    off = align256(off + ((size_t)T + 1) * 4);
    p.off_cursor = off;
    off = align256(off + ((size_t)T + 1) * 4);
    p.off_tmp = off;
    off = align256(off + (size_t)E * C * 4);
    p.bytes = off;
    return p;
}

hipError_t launch_ec_dispatch(const EcPlan &p, const uint16_t *x, int H,
                              const int32_t *token_indices, uint16_t *recv_x, int32_t *tok_off,
                              int32_t *tok_ent, int32_t *num_invalid, char *ws, hipStream_t s)
{
    int32_t *misc = reinterpret_cast<int32_t *>(ws + p.off_misc);
    int32_t *cnt = reinterpret_cast<int32_t *>(ws + p.off_cnt);
    int32_t *cursor = reinterpret_cast<int32_t *>(ws + p.off_cursor);
    int32_t *tmp = reinterpret_cast<int32_t *>(ws + p.off_tmp);
    const int64_t n = (int64_t)p.E * p.C;
    const int W = (p.E + 63) / 64;
    hipError_t err;

    // LDS of the one-block map: the masks, or on the duplicate path T+1
    // counters in the same bytes.
    size_t dyn = (size_t)p.T * W * 8;
    if (dyn < ((size_t)p.T + 1) * 4)
        dyn = ((size_t)p.T + 1) * 4;
    if (p.T > 0 && W == 1 && dyn <= kFusedLds && n <= (int64_t)kInvThreads * kInvRes)
        return launch_fused(x, H, token_indices, p.T, p.C, W, n, dyn, recv_x, tok_off, tok_ent,
                            num_invalid, tmp, s);
    if (dyn + 128 <= (size_t)lds_limit()) {
        if (dyn > 65536) {
            err = hipFuncSetAttribute(reinterpret_cast<const void *>(ec_invert_kernel),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
            if (err != hipSuccess)
                return err;
        }
        hipLaunchKernelGGL(ec_invert_kernel, dim3(1), dim3(kInvThreads), dyn, s, token_indices,
                           p.T, p.C, W, (int)n, 1.0f / (float)p.C, tok_off, tok_ent, num_invalid,
                           tmp);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    } else {
        // misc and cnt are adjacent: one fill clears both
        const int64_t nzero = (int64_t)(p.off_cursor - p.off_misc) / 4;
        hipLaunchKernelGGL(fill_kernel, dim3(grid_for(nzero, 256)), dim3(256), 0, s, misc, nzero,
                           0);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
        hipLaunchKernelGGL(ec_count_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s,
                           token_indices, n, p.T, cnt, misc);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
        hipLaunchKernelGGL(ec_scan_kernel, dim3(1), dim3(kInvThreads), 0, s, cnt, p.T, tok_off,
                           cursor, misc, num_invalid);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
        hipLaunchKernelGGL(ec_place_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s,
                           token_indices, n, p.T, cursor, tmp);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
        hipLaunchKernelGGL(ec_sort_kernel, dim3(p.T), dim3(256), 0, s, tok_off, tmp, tok_ent);
        if ((err = hipGetLastError()) != hipSuccess)
            return err;
    }
    if (p.T == 0)
        return hipSuccess;
    return launch_copy(x, H, token_indices, p.T, n, recv_x, s);
}

}  // namespace ep
