// ep_dispatch.hip -- token dispatch into the receive buffer ("DeepEP-Ascend"
// README, API Overview: dispatch and low_latency_dispatch; Quantization
// Modes in Normal Dispatch: bf16, or float8_e4m3fn codes with float32
// scales).
//
// Token-major: one block per (token, row segment).  The block reads its
// piece of x[t] once into registers (16 bytes per thread per piece), then
// for each of the token's K slots computes the receive row from the layout
// tables and stores the piece there (buffer stores bounded by the row).  The slot arithmetic reads only
// block-uniform addresses, so it runs on the scalar unit.  fp8 quantises
// once per token: a 128-channel group is 16 consecutive lanes; its |max| is
// reduced across them with lane shuffles, the scale is a correctly rounded
// fp32 division, and every element is divided by it (also correctly
// rounded) before the round-to-nearest-even e4m3 encoding.
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

template <int PPT, bool FP8>
__global__ void __launch_bounds__(256)
dispatch_kernel(const uint16_t *__restrict__ x, int H, const int32_t *__restrict__ topk_idx, int K,
                int E, const int32_t *__restrict__ offsets, int padded, int cap_or_rows, int CT,
                int nchunk, const int32_t *__restrict__ chunk_base, const int32_t *__restrict__ local_rank,
                void *__restrict__ recv_x, float *__restrict__ recv_s,
                int32_t *__restrict__ slot_out, int32_t *__restrict__ recv_src,
                int32_t *__restrict__ num_dropped)
{
    const int t = blockIdx.x;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int pieces = H >> 3;
    const int seg0 = blockIdx.y * PPT * bd;
    if (t == 0 && blockIdx.y == 0)
        write_num_dropped(offsets, E, padded, cap_or_rows, num_dropped);

    const char *xrow = reinterpret_cast<const char *>(x) + (size_t)t * H * 2;
    u32x4 v[PPT];
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        int i = seg0 + tid + j * bd;
        v[j] = i < pieces ? ld16(xrow + (size_t)i * 16) : u32x4{0u, 0u, 0u, 0u};
    }

    u32x2 q[FP8 ? PPT : 1];
    float sc[FP8 ? PPT : 1];
    if constexpr (FP8) {
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            int i = seg0 + tid + j * bd;
            float f[8] = {bf16_lo(v[j].x), bf16_hi(v[j].x), bf16_lo(v[j].y), bf16_hi(v[j].y),
                          bf16_lo(v[j].z), bf16_hi(v[j].z), bf16_lo(v[j].w), bf16_hi(v[j].w)};
            float a = 0.0f;
            if (i < pieces)
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    a = fmaxf(a, fabsf(f[u]));
            // 16 lanes = one 128-channel group (pieces and blockDim are multiples of 16)
#pragma unroll
            for (int o = 1; o < 16; o <<= 1)
                a = fmaxf(a, __shfl_xor(a, o, kWave));
            uint32_t c[8];
            if (a == 0.0f) {
                sc[j] = 0.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    c[u] = 0u;
            } else {
                float s = a / 448.0f;
                sc[j] = s;
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    c[u] = f32_to_e4m3_rne(f[u] / s);
            }
            q[j].x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
            q[j].y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        }
    }

    const int c = t / CT;
    const int32_t *trow = topk_idx + (int64_t)t * K;
    const int32_t *rrow = local_rank + (int64_t)t * K;
    const int G = H >> 7;
    for (int k = 0; k < K; ++k) {
        const int e = trow[k];
        int s = -1;
        if ((unsigned)e < (unsigned)E) {
            const int r = chunk_base[(int64_t)e * nchunk + c] + rrow[k];
            if (padded)
                s = r < cap_or_rows ? e * cap_or_rows + r : -1;
            else {
                s = offsets[e] + r;
                if (s >= cap_or_rows)
                    s = -1;
            }
        }
        if (blockIdx.y == 0 && tid == 0) {
            slot_out[(int64_t)t * K + k] = s;
            if (s >= 0 && recv_src)
                recv_src[s] = t;
        }
        if (s < 0)
            continue;
        if constexpr (FP8) {
            const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(recv_x) + (size_t)s * H, H);
            float *sdst = recv_s + (size_t)s * G;
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                int i = seg0 + tid + j * bd;
                row_st8(dst, i * 8, q[j]);
                if ((tid & 15) == 0 && i < pieces)
                    sdst[i >> 4] = sc[j];
            }
        } else {
            const rsrc_t dst = row_rsrc(reinterpret_cast<char *>(recv_x) + (size_t)s * H * 2, H * 2);
#pragma unroll
            for (int j = 0; j < PPT; ++j)
                row_st16(dst, (seg0 + tid + j * bd) * 16, v[j]);
        }
    }
}

// Row pieces per thread and threads per block for a row of `pieces` 16-byte
// pieces: the block size (64..256) that wastes the fewest lanes, up to 8
// pieces per thread, and as many row segments (grid.y) as needed.
struct RowShape {
    int bd, ppt, nseg;
};

RowShape row_shape(int pieces)
{
    RowShape best{64, 1, 1};
    long long best_waste = -1;
    for (int bd : {256, 128, 64}) {
        int ppt = (pieces + bd - 1) / bd;
        if (ppt < 1)
            ppt = 1;
        if (ppt > 8)
            ppt = 8;
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

template <bool FP8>
hipError_t launch_dispatch_t(const LayoutPlan &p, const RowShape &rs, const uint16_t *x, int H,
                             const int32_t *topk_idx, const int32_t *offsets, int padded,
                             int cap_or_rows, void *recv_x, float *recv_s, int32_t *slot,
                             int32_t *recv_src, int32_t *num_dropped, const int32_t *hist,
                             const int32_t *rank, hipStream_t s)
{
    dim3 grid(p.T, rs.nseg), block(rs.bd);
#define EP_DISPATCH_CASE(N)                                                                     \
    case N:                                                                                     \
        hipLaunchKernelGGL((dispatch_kernel<N, FP8>), grid, block, 0, s, x, H, topk_idx, p.K, \
                           p.E, offsets, padded, cap_or_rows, p.CT, p.nchunk, hist, rank,      \
                           recv_x, recv_s,                                                      \
                           slot, recv_src, num_dropped);                                        \
        break;
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
#undef EP_DISPATCH_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const LayoutPlan &p, const uint16_t *x, int H, const int32_t *topk_idx,
                           const int32_t *offsets, bool padded, int cap_or_rows, bool fp8,
                           void *recv_x, float *recv_scales, int32_t *slot, int32_t *recv_src,
                           int32_t *num_dropped, char *ws, hipStream_t s)
{
    const int32_t *hist = reinterpret_cast<const int32_t *>(ws + p.off_hist);
    const int32_t *rank = reinterpret_cast<const int32_t *>(ws + p.off_rank);
    if (p.T == 0) {
        hipLaunchKernelGGL(dropped_only_kernel, dim3(1), dim3(256), 0, s, offsets, p.E,
                           (int)padded, cap_or_rows, num_dropped);
        return hipGetLastError();
    }
    RowShape rs = row_shape(H / 8);
    if (fp8)
        return launch_dispatch_t<true>(p, rs, x, H, topk_idx, offsets, padded, cap_or_rows, recv_x,
                                       recv_scales, slot, recv_src, num_dropped, hist, rank, s);
    return launch_dispatch_t<false>(p, rs, x, H, topk_idx, offsets, padded, cap_or_rows, recv_x,
                                    recv_scales, slot, recv_src, num_dropped, hist, rank, s);
}

}  // namespace ep
