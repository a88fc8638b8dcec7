// ep_api.hip -- the C ABI declared in include/ep.h: argument checks,
// workspace sizing, and stream-ordered launches of the gfx950 kernels.
// Every check happens before anything is enqueued, so a rejected call has
// no effect.  Nothing here touches the GPU except the launches.
#include "ep.h"

#include <hip/hip_runtime.h>

#include "ep_internal.h"

namespace {

constexpr int kMaxExperts = 4096;   // the layout keeps per-expert counts in LDS
constexpr int kMaxRanks = 1024;
constexpr int kMaxTopk = 1024;      // a chunk of the layout holds at least one token's row
constexpr int64_t kI32 = 2147483647LL;
constexpr int kMaxHidden = 1 << 24; // row byte counts and offsets stay 32-bit in the kernels

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

ep_status_t hip_status(hipError_t e) { return e == hipSuccess ? EP_OK : EP_ERR_HIP; }

ep_status_t check_layout_sizes(int T, int K, int E, int R)
{
    if (T < 0 || K < 1 || E < 1 || R < 1)
        return EP_ERR_INVALID_ARG;
    if (E > kMaxExperts || R > kMaxRanks || K > kMaxTopk)
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

ep_status_t ep_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx, int K, int E,
                        const int32_t *offsets, ep_recv_layout_t layout, int cap_or_max_rows,
                        ep_quant_t quant, void *recv_x, void *recv_scales, int32_t *slot,
                        int32_t *recv_src, int32_t *num_dropped, void *ws, size_t ws_bytes,
                        void *stream)
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
    ep::LayoutPlan p = ep::make_layout_plan(T, K, E, 1);
    if ((st = check_ws(ws, ws_bytes, p.bytes)) != EP_OK)
        return st;
    return hip_status(ep::launch_dispatch(p, x, H, topk_idx, offsets, padded, cap_or_max_rows,
                                          (int)quant,
                                          recv_x, recv_scales, slot, recv_src, num_dropped,
                                          static_cast<char *>(ws),
                                          static_cast<hipStream_t>(stream)));
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
