// ep_expert_choice.hip -- expert-choice dispatch ("[Feature Request] Support
// Expert-Choice Routing via Native Expert-Centric API ([num_experts,
// capacity])", Proposed Solutions, Solution 1).
//
// token_indices [E, C] lists, per expert, the tokens it picked.  The copy
// recv[e, c] = x[token_indices[e, c]] is done token-major so each picked x
// row is read from HBM once and written to all of its entries.  That needs
// the inverse map (token -> its flat entries j = e*C + c, ascending), which
// is also the handle that combine walks.  Four launches:
//   1. zero per-token counters;
//   2. count entries per token (integer atomics; order does not matter);
//   3. one block scans the counts into tok_off and cursor starts;
//   4. place each entry at an atomically taken position inside its token's
//      range (an arbitrary order)
// and then one block per token sorts its range into ascending j (each
// value's position is the number of smaller values in the range, so the
// result does not depend on the order step 4 produced) and copies x[t] to
// each of its entries.  No limit on how many experts pick a token.
#include "ep_common.h"
#include "ep_internal.h"

namespace ep {

namespace {

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

// Exclusive scan of cnt[0..T) by one block, ITEMS consecutive values per
// thread per tile, carrying the running total across tiles.
__global__ void __launch_bounds__(1024)
ec_scan_kernel(const int32_t *__restrict__ cnt, int T, int32_t *__restrict__ tok_off,
               int32_t *__restrict__ cursor, const int32_t *__restrict__ ninv_ws,
               int32_t *__restrict__ num_invalid)
{
    constexpr int ITEMS = 8;
    __shared__ int tmp[32];
    int carry = 0;
    const int tile = blockDim.x * ITEMS;
    for (int t0 = 0; t0 < T; t0 += tile) {
        int b = t0 + threadIdx.x * ITEMS;
        int v[ITEMS];
        int sum = 0;
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            v[u] = (b + u < T) ? cnt[b + u] : 0;
            sum += v[u];
        }
        int total;
        int ex = block_exclusive_scan(sum, tmp, &total) + carry;
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            if (b + u < T) {
                tok_off[b + u] = ex;
                cursor[b + u] = ex;
            }
            ex += v[u];
        }
        carry += total;
    }
    if (threadIdx.x == 0) {
        tok_off[T] = carry;
        num_invalid[0] = ninv_ws[0];
    }
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

constexpr int kSortTile = 1024;

template <int PPT>
__global__ void __launch_bounds__(256)
ec_sort_copy_kernel(const uint16_t *__restrict__ x, int H, const int32_t *__restrict__ tok_off,
                    const int32_t *__restrict__ tmp, int32_t *__restrict__ tok_ent,
                    uint16_t *__restrict__ recv)
{
    __shared__ int32_t tile[kSortTile];
    const int t = blockIdx.x;
    const int b = tok_off[t], n = tok_off[t + 1] - b;
    if (n == 0)
        return;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int pieces = H >> 3;
    const int seg0 = blockIdx.y * PPT * bd;

    // copy first: x[t] once into registers, then to every entry (any order)
    const char *xrow = reinterpret_cast<const char *>(x) + (size_t)t * H * 2;
    u32x4 v[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        int i = seg0 + tid + j * bd;
        v[j] = i < pieces ? ld16(xrow + (size_t)i * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    for (int a = 0; a < n; ++a) {
        const int e = tmp[b + a];
        const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(recv) + (size_t)e * H * 2, H * 2);
#pragma unroll
        for (int j = 0; j < PPT; ++j)
            row_st16(dst, (seg0 + tid + j * bd) * 16, v[j]);
    }

    if (blockIdx.y != 0)
        return;
    // rank sort of the token's entries (values are distinct)
    if (n == 1) {
        if (tid == 0)
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

struct RowShape {
    int bd, ppt, nseg;
};

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

int grid_for(int64_t n, int bd)
{
    int64_t g = (n + bd - 1) / bd;
    if (g < 1)
        g = 1;
    if (g > 4096)
        g = 4096;
    return (int)g;
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
    hipError_t err;
    // misc and cnt are adjacent: one fill clears both
    const int64_t nzero = (int64_t)(p.off_cursor - p.off_misc) / 4;
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(nzero, 256)), dim3(256), 0, s, misc, nzero, 0);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    hipLaunchKernelGGL(ec_count_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, token_indices, n,
                       p.T, cnt, misc);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    hipLaunchKernelGGL(ec_scan_kernel, dim3(1), dim3(1024), 0, s, cnt, p.T, tok_off, cursor, misc,
                       num_invalid);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    if (p.T == 0)
        return hipSuccess;
    hipLaunchKernelGGL(ec_place_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, token_indices, n,
                       p.T, cursor, tmp);
    if ((err = hipGetLastError()) != hipSuccess)
        return err;
    RowShape rs = row_shape(H / 8, 8);
    dim3 grid(p.T, rs.nseg), block(rs.bd);
#define EP_EC_CASE(N)                                                                           \
    case N:                                                                                     \
        hipLaunchKernelGGL((ec_sort_copy_kernel<N>), grid, block, 0, s, x, H, tok_off, tmp,   \
                           tok_ent, recv_x);                                                    \
        break;
    switch (rs.ppt) {
        EP_EC_CASE(1)
        EP_EC_CASE(2)
        EP_EC_CASE(3)
        EP_EC_CASE(4)
        EP_EC_CASE(5)
        EP_EC_CASE(6)
        EP_EC_CASE(7)
        EP_EC_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef EP_EC_CASE
    return hipGetLastError();
}

}  // namespace ep
