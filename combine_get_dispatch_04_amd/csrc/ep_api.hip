// ep_api.hip -- the C ABI declared in include/ep.h: argument checks,
// workspace sizing, and stream-ordered launches of the gfx950 kernels.
// Every check happens before anything is enqueued, so a rejected call has
// no effect.  Nothing here touches the GPU except the launches.
#include "ep.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "ep_internal.h"

namespace {

constexpr int kMaxExperts = 4096;   // the layout keeps per-expert counts in LDS
constexpr int kMaxRanks = 1024;
constexpr int64_t kI32 = 2147483647LL;
constexpr int kMaxHidden = 1 << 24; // row byte counts and offsets stay 32-bit in the kernels

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ep_status_t hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

ep_status_t check_layout_sizes(int T, int K, int E, int R)
{
    if (T < 0 || K < 1 || E < 1 || R < 1)
        return EP_ERR_INVALID_ARG;
    if (E > kMaxExperts || R > kMaxRanks)
        return EP_ERR_UNSUPPORTED;
    if (E % R != 0)
        return EP_ERR_INVALID_ARG;
    if ((int64_t)T * K > kI32)
        return EP_ERR_INVALID_ARG;
    return EP_OK;
}

ep_status_t check_ws(const void *ws, size_t ws_bytes, size_t need)
{
    if (!ws || !aligned(ws, 256) || ws_bytes < need)
        return EP_ERR_WORKSPACE;
    return EP_OK;
}

// The arguments of a dispatch (ep_dispatch and the no-allocation form),
// other than the workspace.
ep_status_t check_dispatch_args(const uint16_t *x, int T, int H, const int32_t *topk_idx, int K,
                                int E, const int32_t *offsets, ep_recv_layout_t layout,
                                int cap_or_max_rows, ep_quant_t quant, const void *recv_x,
                                const void *recv_scales, const int32_t *slot,
                                const int32_t *recv_src, const int32_t *num_dropped)
{
    ep_status_t st = check_layout_sizes(T, K, E, 1);
    if (st != EP_OK)
        return st;
    if (layout != EP_LAYOUT_CONTIGUOUS && layout != EP_LAYOUT_PADDED)
        return EP_ERR_INVALID_ARG;
    if ((int)quant < (int)EP_QUANT_BF16 || (int)quant > (int)EP_QUANT_MXFP4_E2M1)
        return EP_ERR_INVALID_ARG;
    const bool quantised = quant != EP_QUANT_BF16;
    const bool mx = quant == EP_QUANT_MXFP8_E4M3 || quant == EP_QUANT_MXFP8_E5M2 ||
                    quant == EP_QUANT_MXFP4_E2M1;
    const bool padded = layout == EP_LAYOUT_PADDED;
    if (H < 8 || H % 8 != 0 || (quant == EP_QUANT_FP8_E4M3_G128 && H % 128 != 0) ||
        (mx && H % 32 != 0))
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (cap_or_max_rows < 0)
        return EP_ERR_INVALID_ARG;
    const int64_t rows = padded ? (int64_t)E * cap_or_max_rows : cap_or_max_rows;
    if (rows > kI32)
        return EP_ERR_INVALID_ARG;
    if (!offsets || !num_dropped || (T > 0 && (!x || !topk_idx || !slot)) ||
        (rows > 0 && T > 0 && !recv_x) || (quantised && rows > 0 && T > 0 && !recv_scales))
        return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || (!mx && !aligned(recv_scales, 4)) ||
        !aligned(topk_idx, 4) || !aligned(offsets, 4) || !aligned(slot, 4) ||
        !aligned(recv_src, 4) || !aligned(num_dropped, 4))
        return EP_ERR_INVALID_ARG;
    return EP_OK;
}

// Scratch of ep_layout_dispatch_noalloc: the layout's per-chunk tables and
// per-entry ranks, which the dispatch then reads (what the workspace holds
// for the pair).  Each device holds its own copy for the life of the
// process.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): it uses the device address
// that hipGetSymbolAddress returned for the device, taken once per device
// with that device current.
__device__ __align__(256) char scratch[EP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the device that runs `stream`, or
// nullptr if the runtime cannot give it.
char *scratch_for(hipStream_t stream)
{
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    dev = cur;
    if (stream && (hipStreamGetDevice(stream, &dev) != hipSuccess)) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur)
            (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        addr[dev] = p;
    }
    return static_cast<char *>(addr[dev]);
}

}  // namespace

extern "C" {

const char *ep_status_string(ep_status_t status)
{
    switch (status) {
    case EP_OK:
        return "ok";
    case EP_ERR_INVALID_ARG:
        return "invalid argument";
    case EP_ERR_UNSUPPORTED:
        return "unsupported size or mode";
    case EP_ERR_WORKSPACE:
        return "workspace missing, misaligned or too small";
    case EP_ERR_HIP:
        return "HIP launch error";
    }
    return "unknown status";
}

size_t ep_workspace_bytes(int T, int K, int E, int R)
{
    if (check_layout_sizes(T, K, E, R) != EP_OK)
        return 0;
    return ep::make_layout_plan(T, K, E, R).bytes;
}

size_t ep_ec_workspace_bytes(int T, int E, int C)
{
    if (T < 0 || E < 1 || C < 1 || (int64_t)E * C > kI32 || T >= kI32)
        return 0;
    return ep::make_ec_plan(T, E, C).bytes;
}

ep_status_t ep_get_dispatch_layout(const int32_t *topk_idx, int T, int K, int E, int R,
                                   int32_t *counts, int32_t *offsets, int32_t *tokens_per_rank,
                                   uint8_t *is_token_in_rank, int32_t *num_invalid, void *ws,
                                   size_t ws_bytes, void *stream)
{
    ep_status_t st = check_layout_sizes(T, K, E, R);
    if (st != EP_OK)
        return st;
    if ((T > 0 && !topk_idx) || !counts || !offsets || !num_invalid)
        return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
        !aligned(tokens_per_rank, 4) || !aligned(num_invalid, 4))
        return EP_ERR_INVALID_ARG;
    ep::LayoutPlan p = ep::make_layout_plan(T, K, E, R);
    if ((st = check_ws(ws, ws_bytes, p.bytes)) != EP_OK)
        return st;
    return hip_status(ep::launch_layout(p, topk_idx, counts, offsets, tokens_per_rank,
                                        is_token_in_rank, num_invalid, static_cast<char *>(ws),
                                        static_cast<hipStream_t>(stream)));
}

size_t ep_workspace_bytes_rounds(int T, int K, int E, int R, int round_tokens)
{
    if (check_layout_sizes(T, K, E, R) != EP_OK || round_tokens < 1)
        return 0;
    const int rt = round_tokens < T ? round_tokens : T;
    if (rt == 0)
        return ep::make_layout_plan(0, K, E, R).bytes;
    const int full = T / rt, last = T - full * rt;
    const size_t stride = ep::make_layout_plan(rt, K, E, R).bytes;
    return stride * (size_t)full + (last ? ep::make_layout_plan(last, K, E, R).bytes : 0);
}

ep_status_t ep_get_dispatch_layout_rounds(const int32_t *topk_idx, int T, int K, int E, int R,
                                          int round_tokens, int32_t *counts, int32_t *offsets,
                                          int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                                          int32_t *num_invalid, void *ws, size_t ws_bytes,
                                          void *stream)
{
    ep_status_t st = check_layout_sizes(T, K, E, R);
    if (st != EP_OK)
        return st;
    if (round_tokens < 1)
        return EP_ERR_INVALID_ARG;
    if ((T > 0 && !topk_idx) || !counts || !offsets || !num_invalid)
        return EP_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
        !aligned(tokens_per_rank, 4) || !aligned(num_invalid, 4))
        return EP_ERR_INVALID_ARG;
    if ((st = check_ws(ws, ws_bytes, ep_workspace_bytes_rounds(T, K, E, R, round_tokens))) !=
        EP_OK)
        return st;
    if (T == 0)
        return EP_OK;                       // no rounds: nothing to write
    const int rt = round_tokens < T ? round_tokens : T;
    const int full = T / rt, last = T - full * rt;
    const ep::LayoutPlan p = ep::make_layout_plan(rt, K, E, R);
    const size_t stride = p.bytes;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(ws);
    // the full rounds, at most 65535 per launch pair (grid.y / grid.x)
    for (int r0 = 0; r0 < full; r0 += 65535) {
        const int n = full - r0 < 65535 ? full - r0 : 65535;
        hipError_t e = ep::launch_layout(
            p, topk_idx + (int64_t)r0 * rt * K, counts + (int64_t)r0 * E,
            offsets + (int64_t)r0 * (E + 1), tokens_per_rank ? tokens_per_rank + (int64_t)r0 * R : nullptr,
            is_token_in_rank ? is_token_in_rank + (int64_t)r0 * rt * R : nullptr,
            num_invalid + r0, w + stride * (size_t)r0, s, n, stride);
        if (e != hipSuccess)
            return EP_ERR_HIP;
    }
    if (last) {
        const ep::LayoutPlan pl = ep::make_layout_plan(last, K, E, R);
        const int64_t t0 = (int64_t)full * rt;
        return hip_status(ep::launch_layout(
            pl, topk_idx + t0 * K, counts + (int64_t)full * E, offsets + (int64_t)full * (E + 1),
            tokens_per_rank ? tokens_per_rank + (int64_t)full * R : nullptr,
            is_token_in_rank ? is_token_in_rank + t0 * R : nullptr, num_invalid + full,
            w + stride * (size_t)full, s));
    }
    return EP_OK;
}

ep_status_t ep_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx, int K, int E,
                        const int32_t *offsets, ep_recv_layout_t layout, int cap_or_max_rows,
                        ep_quant_t quant, void *recv_x, void *recv_scales, int32_t *slot,
                        int32_t *recv_src, int32_t *num_dropped, void *ws, size_t ws_bytes,
                        void *stream)
{
    ep_status_t st = check_dispatch_args(x, T, H, topk_idx, K, E, offsets, layout,
                                         cap_or_max_rows, quant, recv_x, recv_scales, slot,
                                         recv_src, num_dropped);
    if (st != EP_OK)
        return st;
    ep::LayoutPlan p = ep::make_layout_plan(T, K, E, 1);
    if ((st = check_ws(ws, ws_bytes, p.bytes)) != EP_OK)
        return st;
    return hip_status(ep::launch_dispatch(p, x, H, topk_idx, offsets,
                                          layout == EP_LAYOUT_PADDED, cap_or_max_rows,
                                          (int)quant,
                                          recv_x, recv_scales, slot, recv_src, num_dropped,
                                          static_cast<char *>(ws),
                                          static_cast<hipStream_t>(stream)));
}

ep_status_t ep_layout_dispatch_noalloc(const uint16_t *x, int T, int H, const int32_t *topk_idx,
                                       int K, int E, int R, int32_t *counts, int32_t *offsets,
                                       int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                                       int32_t *num_invalid, ep_recv_layout_t layout,
                                       int cap_or_max_rows, ep_quant_t quant, void *recv_x,
                                       void *recv_scales, int32_t *slot, int32_t *recv_src,
                                       int32_t *num_dropped, void *stream)
{
    // every check of ep_get_dispatch_layout and ep_dispatch, then the size
    // check, all before anything is enqueued
    ep_status_t st = check_layout_sizes(T, K, E, R);
    if (st != EP_OK)
        return st;
    if ((T > 0 && !topk_idx) || !counts || !offsets || !num_invalid)
        return EP_ERR_INVALID_ARG;
    if (!aligned(counts, 4) || !aligned(tokens_per_rank, 4) || !aligned(num_invalid, 4))
        return EP_ERR_INVALID_ARG;
    st = check_dispatch_args(x, T, H, topk_idx, K, E, offsets, layout, cap_or_max_rows, quant,
                             recv_x, recv_scales, slot, recv_src, num_dropped);
    if (st != EP_OK)
        return st;
    const ep::LayoutPlan pl = ep::make_layout_plan(T, K, E, R);
    const ep::LayoutPlan pd = ep::make_layout_plan(T, K, E, 1);
    if (pl.bytes > EP_NOALLOC_SCRATCH_BYTES || pd.bytes > EP_NOALLOC_SCRATCH_BYTES)
        return EP_ERR_UNSUPPORTED;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = scratch_for(s);
    if (!ws)
        return EP_ERR_HIP;
    // the layout writes every table entry the dispatch reads, so the
    // scratch needs no clearing between calls
    hipError_t e = ep::launch_layout(pl, topk_idx, counts, offsets, tokens_per_rank,
                                     is_token_in_rank, num_invalid, ws, s);
    if (e != hipSuccess)
        return EP_ERR_HIP;
    return hip_status(ep::launch_dispatch(pd, x, H, topk_idx, offsets,
                                          layout == EP_LAYOUT_PADDED, cap_or_max_rows,
                                          (int)quant, recv_x, recv_scales, slot, recv_src,
                                          num_dropped, ws, s));
}

ep_status_t ep_low_latency_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx,
                                    int K, int E, int cap, ep_quant_t quant, void *recv_x,
                                    void *recv_scales, int32_t *slot, int32_t *recv_src,
                                    int32_t *recv_count, int32_t *num_dropped,
                                    int32_t *num_invalid, void *stream)
{
    ep_status_t st = check_layout_sizes(T, K, E, 1);
    if (st != EP_OK)
        return st;
    if ((int)quant < (int)EP_QUANT_BF16 || (int)quant > (int)EP_QUANT_MXFP4_E2M1)
        return EP_ERR_INVALID_ARG;
    const bool quantised = quant != EP_QUANT_BF16;
    const bool mx = quant == EP_QUANT_MXFP8_E4M3 || quant == EP_QUANT_MXFP8_E5M2 ||
                    quant == EP_QUANT_MXFP4_E2M1;
    if (H < 8 || H % 8 != 0 || (quant == EP_QUANT_FP8_E4M3_G128 && H % 128 != 0) ||
        (mx && H % 32 != 0))
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (cap < 0 || (int64_t)E * cap > kI32)
        return EP_ERR_INVALID_ARG;
    if (!ep::ll_dispatch_fits(T, K, H, (int)quant))
        return EP_ERR_UNSUPPORTED;
    const bool rows = (int64_t)E * cap > 0;
    if (!recv_count || !num_dropped || !num_invalid || (T > 0 && (!x || !topk_idx || !slot)) ||
        (rows && T > 0 && !recv_x) || (quantised && rows && T > 0 && !recv_scales))
        return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || (!mx && !aligned(recv_scales, 4)) ||
        !aligned(topk_idx, 4) || !aligned(slot, 4) || !aligned(recv_src, 4) ||
        !aligned(recv_count, 4) || !aligned(num_dropped, 4) || !aligned(num_invalid, 4))
        return EP_ERR_INVALID_ARG;
    return hip_status(ep::launch_ll_dispatch(x, T, H, topk_idx, K, E, cap, (int)quant, recv_x,
                                             recv_scales, slot, recv_src, recv_count,
                                             num_dropped, num_invalid,
                                             static_cast<hipStream_t>(stream)));
}

ep_status_t ep_combine(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                       const float *topk_weights, int T, int K, uint16_t *out, void *stream)
{
    if (T < 0 || K < 1 || H < 8 || H % 8 != 0 || (int64_t)T * K > kI32 || y_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (T > 0 && (!slot || !out || (y_rows > 0 && !y)))
        return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(slot, 4) || !aligned(topk_weights, 4))
        return EP_ERR_INVALID_ARG;
    return hip_status(ep::launch_combine(y, y_rows, H, slot, topk_weights, T, K, out,
                                         static_cast<hipStream_t>(stream)));
}

size_t ep_pack_workspace_bytes(int T, int K, int E, int R)
{
    if (check_layout_sizes(T, K, E, R) != EP_OK)
        return 0;
    return ep::make_rank_plan(T, K, E, R).bytes;
}

ep_status_t ep_pack_by_rank(const uint16_t *x, int T, int H, const int32_t *topk_idx,
                            const float *topk_weights, int K, int E, int R, int max_rows,
                            int32_t *tokens_per_rank, int32_t *rank_offsets, uint16_t *send_x,
                            int32_t *send_src, int32_t *send_idx, float *send_w,
                            int32_t *pack_pos, int32_t *num_dropped, void *ws, size_t ws_bytes,
                            void *stream)
{
    ep_status_t st = check_layout_sizes(T, K, E, R);
    if (st != EP_OK)
        return st;
    if (H < 8 || H % 8 != 0 || max_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (!tokens_per_rank || !rank_offsets || !num_dropped ||
        (T > 0 && (!x || !topk_idx || !pack_pos)) ||
        (T > 0 && max_rows > 0 && (!send_x || !send_src || !send_idx)))
        return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(send_x, 16) || !aligned(topk_idx, 4) ||
        !aligned(topk_weights, 4) || !aligned(tokens_per_rank, 4) || !aligned(rank_offsets, 4) ||
        !aligned(send_src, 4) || !aligned(send_idx, 4) || !aligned(send_w, 4) ||
        !aligned(pack_pos, 4) || !aligned(num_dropped, 4))
        return EP_ERR_INVALID_ARG;
    if ((int64_t)T * R > kI32 || (int64_t)max_rows * K > kI32)
        return EP_ERR_INVALID_ARG;
    const ep::RankPlan rp = ep::make_rank_plan(T, K, E, R);
    if ((st = check_ws(ws, ws_bytes, rp.bytes)) != EP_OK)
        return st;
    return hip_status(ep::launch_rank_pack(rp, x, H, topk_idx, topk_weights, E, R, max_rows,
                                           tokens_per_rank, rank_offsets, send_x, send_src,
                                           send_idx, send_w, pack_pos, num_dropped,
                                           static_cast<char *>(ws),
                                           static_cast<hipStream_t>(stream)));
}

ep_status_t ep_combine_partial(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                               const float *weights, int S, int K, float *partial, void *stream)
{
    if (S < 0 || K < 1 || H < 8 || H % 8 != 0 || (int64_t)S * K > kI32 || y_rows < 0)
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (S > 0 && (!slot || !partial || (y_rows > 0 && !y)))
        return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(partial, 16) || !aligned(slot, 4) || !aligned(weights, 4))
        return EP_ERR_INVALID_ARG;
    return hip_status(ep::launch_combine_partial(y, y_rows, H, slot, weights, S, K, partial,
                                                 static_cast<hipStream_t>(stream)));
}

ep_status_t ep_combine_ranks(const float *partial, int rows, int H, const int32_t *pack_pos,
                             int T, int R, uint16_t *out, void *stream)
{
    if (T < 0 || R < 1 || rows < 0 || H < 8 || H % 8 != 0 || (int64_t)T * R > kI32)
        return EP_ERR_INVALID_ARG;
    if (R > kMaxRanks || H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (T > 0 && (!pack_pos || !out || (rows > 0 && !partial)))
        return EP_ERR_INVALID_ARG;
    if (!aligned(partial, 16) || !aligned(out, 16) || !aligned(pack_pos, 4))
        return EP_ERR_INVALID_ARG;
    return hip_status(ep::launch_rank_sum(partial, rows, H, pack_pos, T, R, out,
                                          static_cast<hipStream_t>(stream)));
}

ep_status_t ep_dispatch_expert_choice(const uint16_t *x, int T, int H,
                                      const int32_t *token_indices, int E, int C,
                                      uint16_t *recv_x, int32_t *tok_off, int32_t *tok_ent,
                                      int32_t *num_invalid, void *ws, size_t ws_bytes,
                                      void *stream)
{
    if (T < 0 || T >= kI32 || E < 1 || C < 1 || (int64_t)E * C > kI32 || H < 8 || H % 8 != 0)
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (!token_indices || !tok_off || !tok_ent || !num_invalid || !recv_x || (T > 0 && !x))
        return EP_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(token_indices, 4) ||
        !aligned(tok_off, 4) || !aligned(tok_ent, 4) || !aligned(num_invalid, 4))
        return EP_ERR_INVALID_ARG;
    ep::EcPlan p = ep::make_ec_plan(T, E, C);
    ep_status_t st = check_ws(ws, ws_bytes, p.bytes);
    if (st != EP_OK)
        return st;
    return hip_status(ep::launch_ec_dispatch(p, x, H, token_indices, recv_x, tok_off, tok_ent,
                                             num_invalid, static_cast<char *>(ws),
                                             static_cast<hipStream_t>(stream)));
}

ep_status_t ep_combine_expert_choice(const uint16_t *y, const float *weights, int E, int C, int H,
                                     const int32_t *tok_off, const int32_t *tok_ent, int T,
                                     uint16_t *out, void *stream)
{
    if (T < 0 || T >= kI32 || E < 1 || C < 1 || (int64_t)E * C > kI32 || H < 8 || H % 8 != 0)
        return EP_ERR_INVALID_ARG;
    if (H > kMaxHidden)
        return EP_ERR_UNSUPPORTED;
    if (T > 0 && (!y || !weights || !tok_off || !tok_ent || !out))
        return EP_ERR_INVALID_ARG;
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(weights, 4) || !aligned(tok_off, 4) ||
        !aligned(tok_ent, 4))
        return EP_ERR_INVALID_ARG;
    return hip_status(ep::launch_ec_combine(y, weights, E, C, H, tok_off, tok_ent, T, out,
                                            static_cast<hipStream_t>(stream)));
}

}  // extern "C"
