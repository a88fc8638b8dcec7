// ep_rank.hip -- one rank's share of the expert-parallel exchange
// ("DeepEP-Ascend" README, API Overview: get_dispatch_layout returns
// num_tokens_per_rank and is_token_in_rank; dispatch sends each token to the
// ranks of its experts; combine reduces what comes back).  Rank r owns
// experts [r*E/R, (r+1)*E/R).
//
// Sender pack: a stable counting sort keyed by (destination rank, token).
// The layout kernels run with rank keys (ep_layout.hip): an entry is keyed
// by its expert's rank when it is the first of its token's valid entries on
// that rank, so the counts are the tokens per rank, the offsets the start of
// each rank's rows, and each key entry's chunk base + local rank its place
// among the rank's tokens.  rank_pack_kernel is then token-major, like the
// dispatch: one block per (token, row segment) reads its piece of x[t] once
// into registers, finds the token's packed rows one per lane (the same
// first-on-rank test as the layout), and stores the piece to each of them;
// wave 0 of row segment 0 writes the handle (pack_pos), the source token and
// the row's entries for that rank (local expert ids, -1 elsewhere) with
// their weights.
//
// Sender sum: after the receivers' partial combines (ep_combine.hip, fp32
// rows) come back, rank_sum_kernel adds a token's partial rows in rank order
// with fp32 adds and rounds once to bf16 (nearest even).
#include "ep_common.h"
#include "ep_internal.h"

namespace ep {

namespace {

// One block per (token, row segment), PPT 16-byte pieces per thread.
template <int PPT>
__global__ void __launch_bounds__(256)
rank_pack_kernel(const uint16_t *__restrict__ x, int H, const int32_t *__restrict__ topk_idx,
                 const float *__restrict__ w, int K, int E, int R, int per_rank,
                 const int32_t *__restrict__ offsets, int max_rows, int CT, int CE, int nchunk,
                 const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ local_rank,
                 uint16_t *__restrict__ send_x, int32_t *__restrict__ send_src,
                 int32_t *__restrict__ send_idx, float *__restrict__ send_w,
                 int32_t *__restrict__ pack_pos, int32_t *__restrict__ num_dropped)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int lane = tid & (kWave - 1);
    const int pieces = H >> 3;
    const int seg0 = blockIdx.y * PPT * bd;
    const bool writer = blockIdx.y == 0 && tid < kWave;
    if (t == 0 && blockIdx.y == 0 && tid == 0) {
        const int n = offsets[R];
        num_dropped[0] = n > max_rows ? n - max_rows : 0;
    }

    const char *xrow = reinterpret_cast<const char *>(x) + (size_t)t * H * 2;
    u32x4 v[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = seg0 + tid + j * bd;
        v[j] = i < pieces ? ld16(xrow + (size_t)i * 16) : u32x4{0u, 0u, 0u, 0u};
    }

    const int c = t / CT;
    const int32_t *trow = topk_idx + (int64_t)t * K;
    const int32_t *rrow = local_rank + (int64_t)t * K;
    const float *wrow = w ? w + (int64_t)t * K : nullptr;
    const int64_t rb = 2 * (int64_t)H;
    for (int k0 = 0; k0 < K; k0 += kWave) {
        const int k = k0 + lane;
        const int kn = K - k0 < kWave ? K - k0 : kWave;
        const int e = k < K ? trow[k] : -1;
        const int r = (unsigned)e < (unsigned)E ? e / per_rank : -1;
        // first of the token's valid entries on rank r: none of the earlier
        // lanes of this round, nor of earlier rounds, is on r
        bool first = r >= 0;
        for (int kk = 0; kk < kn; ++kk) {
            const int rk = __builtin_amdgcn_readlane(r, kk);
            first = first && !(kk < lane && rk == r);
        }
        for (int k2 = 0; first && k2 < k0; ++k2) {
            const int e2 = trow[k2];
            if ((unsigned)e2 < (unsigned)E && e2 / per_rank == r)
                first = false;
        }
        int sl = -1;
        if (first) {
            // rows longer than a layout chunk: each entry's own chunk
            const int ck = CE > 0 ? (int)(((int64_t)t * K + k) / CE) : c;
            const int p = offsets[r] + chunk_base[(int64_t)r * nchunk + ck] + rrow[k];
            sl = p < max_rows ? p : -1;
            if (writer) {
                pack_pos[(int64_t)t * R + r] = sl;
                if (sl >= 0)
                    send_src[sl] = t;
            }
        }
        for (int kk = 0; kk < kn; ++kk) {
            const int s = __builtin_amdgcn_readlane(sl, kk);
            if (s < 0)
                continue;
            const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(send_x) + (size_t)s * rb, (int)rb);
#pragma unroll
            for (int j = 0; j < PPT; ++j)
                row_st16(dst, (seg0 + tid + j * bd) * 16, v[j]);
            if (writer) {
                // the row's entries for this rank: local ids, -1 elsewhere
                const int rr = __builtin_amdgcn_readlane(r, kk);
                for (int j0 = 0; j0 < K; j0 += kWave) {
                    const int jj = j0 + lane;
                    if (jj >= K)
                        break;
                    const int ej = trow[jj];
                    const bool here = (unsigned)ej < (unsigned)E && ej / per_rank == rr;
                    send_idx[(int64_t)s * K + jj] = here ? ej - rr * per_rank : -1;
                    if (send_w)
                        send_w[(int64_t)s * K + jj] = here ? (wrow ? wrow[jj] : 1.0f) : 0.0f;
                }
            }
        }
    }
    // ranks the token is not sent to
    if (writer) {
        for (int r0 = 0; r0 < R; r0 += kWave) {
            const int rr = r0 + lane;
            if (rr >= R)
                break;
            bool present = false;
            for (int k = 0; k < K && !present; ++k) {
                const int e = trow[k];
                present = (unsigned)e < (unsigned)E && e / per_rank == rr;
            }
            if (!present)
                pack_pos[(int64_t)t * R + rr] = -1;
        }
    }
}

// With no tokens only the drop counter is written.
__global__ void rank_pack_empty_kernel(const int32_t *__restrict__ offsets, int R, int max_rows,
                                       int32_t *__restrict__ num_dropped)
{
    if (threadIdx.x == 0) {
        const int n = offsets[R];
        num_dropped[0] = n > max_rows ? n - max_rows : 0;
    }
}

// One block per (token, row segment); a thread owns PPT units of 4 channels
// (16 bytes of fp32 partials, 8 bytes of output), so that each load
// instruction of a wave reads 1 KiB of a row with no gaps.  Each round takes
// the token's next G valid rows in rank order (one load of 64 positions per
// wave, a ballot, readlane), requests all of their pieces, then adds them in
// order.
template <int PPT, int G>
__global__ void __launch_bounds__(256)
rank_sum_kernel(const float *__restrict__ partial, int rows, int H,
                const int32_t *__restrict__ pack_pos, int R, uint16_t *__restrict__ out)
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
    const int32_t *prow = pack_pos + (int64_t)t * R;
    const int rbytes = units * 16;
    for (int r0 = 0; r0 < R; r0 += kWave) {
        const int rr = r0 + lane;
        const int pv = rr < R ? prow[rr] : -1;
        uint64_t m = ballot((unsigned)pv < (unsigned)rows);
        while (m) {
            int sel[G];
            bool ok[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                ok[g] = m != 0;
                const int b = ok[g] ? (int)__builtin_ctzll(m) : 0;
                m &= m - 1;
                sel[g] = ok[g] ? __builtin_amdgcn_readlane(pv, b) : 0;
            }
            u32x4 v[G][PPT];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const rsrc_t src = row_rsrc(reinterpret_cast<const char *>(partial) +
                                                (size_t)sel[g] * rbytes,
                                            ok[g] ? rbytes : 0);
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
                    acc[j][0] += __uint_as_float(v[g][j].x);
                    acc[j][1] += __uint_as_float(v[g][j].y);
                    acc[j][2] += __uint_as_float(v[g][j].z);
                    acc[j][3] += __uint_as_float(v[g][j].w);
                }
            }
        }
    }
    // sc1 stores (the receive rows' policy): 135.4-136.1 -> 133.1-133.3 us at
    // R = 8, 92.2-92.3 -> 90.4-90.8 at R = 4
    const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(out) + (size_t)t * H * 2, units * 8);
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int i = seg0 + threadIdx.x + j * blockDim.x;
        if (i < units)
            row_st8(dst, i * 8,
                    u32x2{pack_bf16x2(acc[j][0], acc[j][1]), pack_bf16x2(acc[j][2], acc[j][3])});
    }
}

struct Shape {
    int bd, ppt, nseg;
};

// The block size (64..256) that leaves the fewest lanes idle, with at most
// maxppt units per thread, and as many row segments as needed.
Shape shape_for(int units, int maxppt)
{
    Shape best{64, 1, 1};
    long long best_waste = -1;
    for (int bd : {256, 128, 64}) {
        int ppt = (units + bd - 1) / bd;
        ppt = ppt < 1 ? 1 : (ppt > maxppt ? maxppt : ppt);
        int nseg = (units + ppt * bd - 1) / (ppt * bd);
        nseg = nseg < 1 ? 1 : nseg;
        const long long waste = (long long)nseg * ppt * bd - units;
        if (best_waste < 0 || waste < best_waste) {
            best = {bd, ppt, nseg};
            best_waste = waste;
        }
    }
    return best;
}

}  // namespace

hipError_t launch_rank_pack(const RankPlan &rp, const uint16_t *x, int H, const int32_t *topk_idx,
                            const float *w, int E, int R, int max_rows, int32_t *tokens_per_rank,
                            int32_t *rank_offsets, uint16_t *send_x, int32_t *send_src,
                            int32_t *send_idx, float *send_w, int32_t *pack_pos,
                            int32_t *num_dropped, char *ws, hipStream_t s)
{
    const LayoutPlan &p = rp.lp;
    int32_t *ninv = reinterpret_cast<int32_t *>(ws + rp.off_misc);
    hipError_t err = launch_layout(p, topk_idx, tokens_per_rank, rank_offsets, nullptr, nullptr,
                                   ninv, ws, s);
    if (err != hipSuccess)
        return err;
    if (p.T == 0) {
        hipLaunchKernelGGL(rank_pack_empty_kernel, dim3(1), dim3(64), 0, s, rank_offsets, R,
                           max_rows, num_dropped);
        return hipGetLastError();
    }
    const int32_t *hist = reinterpret_cast<const int32_t *>(ws + p.off_hist);
    const int32_t *rank = reinterpret_cast<const int32_t *>(ws + p.off_rank);
    // as the bf16 dispatch: up to 8 pieces per thread, 2 for few tokens
    const Shape sh = shape_for(H / 8, p.T < 1024 ? 2 : 8);
    if ((uint64_t)p.T * sh.bd > 0xFFFFFFFFull)
        return hipErrorInvalidConfiguration;
    dim3 grid(p.T, sh.nseg), block(sh.bd);
#define EP_PACK_CASE(N)                                                                           \
    case N:                                                                                       \
        hipLaunchKernelGGL((rank_pack_kernel<N>), grid, block, 0, s, x, H, topk_idx, w, p.K, E, R, \
                           E / R, rank_offsets, max_rows, p.CT, p.CE, p.nchunk, hist, rank,       \
                           send_x,                                                                \
                           send_src, send_idx, send_w, pack_pos, num_dropped);                    \
        break;
    switch (sh.ppt) {
        EP_PACK_CASE(1)
        EP_PACK_CASE(2)
        EP_PACK_CASE(3)
        EP_PACK_CASE(4)
        EP_PACK_CASE(5)
        EP_PACK_CASE(6)
        EP_PACK_CASE(7)
        EP_PACK_CASE(8)
    default:
        return hipErrorInvalidValue;
    }
#undef EP_PACK_CASE
    return hipGetLastError();
}

hipError_t launch_rank_sum(const float *partial, int rows, int H, const int32_t *pack_pos, int T,
                           int R, uint16_t *out, hipStream_t s)
{
    if (T == 0)
        return hipSuccess;
    // Units of 4 channels, at most 4 per thread, 8 rows requested per round.
    const Shape sh = shape_for(H / 4, 4);
    if ((uint64_t)T * sh.bd > 0xFFFFFFFFull)
        return hipErrorInvalidConfiguration;
    dim3 grid(T, sh.nseg), block(sh.bd);
    switch (sh.ppt) {
    case 1:
        hipLaunchKernelGGL((rank_sum_kernel<1, 8>), grid, block, 0, s, partial, rows, H, pack_pos,
                           R, out);
        break;
    case 2:
        hipLaunchKernelGGL((rank_sum_kernel<2, 8>), grid, block, 0, s, partial, rows, H, pack_pos,
                           R, out);
        break;
    case 3:
        hipLaunchKernelGGL((rank_sum_kernel<3, 8>), grid, block, 0, s, partial, rows, H, pack_pos,
                           R, out);
        break;
    default:
        hipLaunchKernelGGL((rank_sum_kernel<4, 8>), grid, block, 0, s, partial, rows, H, pack_pos,
                           R, out);
        break;
    }
    return hipGetLastError();
}

}  // namespace ep
