// ep_internal.h -- host-side plans and launchers shared by the libep sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// How the layout splits topk_idx: blocks ("chunks") of CT whole tokens.
// Inside a chunk, `waves` waves each take a contiguous run of entries.
struct LayoutPlan {
    int T, K, E, R;
    int CT;        // tokens per chunk
    int CE;        // entries per chunk when a row is longer than a chunk (rows
                   // then span chunks), else 0
    int nchunk;    // ceil(T / CT)
    int waves;     // waves per chunk block
    int epl;       // entries per lane (1..32, a power of two)
    int nbits;     // bits needed for an expert id in [0, E)
    // rank keys (the sender pack): E counts ranks, the entries hold experts
    // in [0, key_experts), key_div per rank; key_div == 0 for expert keys
    int key_experts, key_div;
    size_t lds;    // dynamic shared memory of the chunk kernel
    // workspace carve-up (byte offsets, 256-aligned)
    // off_tamax: [T] fp32 row maxima for the per-token modes when a row spans
    // several dispatch blocks
    size_t off_hist, off_rank, off_rpart, off_ipart, off_tamax, bytes;
};

LayoutPlan make_layout_plan(int T, int K, int E, int R);

// The layout of the sender pack: rank keys over R ranks of E/R experts each,
// plus room for its invalid-entry count (off_misc) in the workspace.
struct RankPlan {
    LayoutPlan lp;
    size_t off_misc, bytes;
};
RankPlan make_rank_plan(int T, int K, int E, int R);

struct EcPlan {
    int T, E, C;
    size_t off_cnt, off_cursor, off_tmp, off_misc, bytes;
};
EcPlan make_ec_plan(int T, int E, int C);

// `rounds` > 1: that many rounds of p.T tokens side by side (topk_idx,
// is_token_in_rank and the per-round outputs consecutive), round r's tables
// at ws + r * round_bytes (a multiple of 256).
hipError_t launch_layout(const LayoutPlan &p, const int32_t *topk_idx, int32_t *counts,
                         int32_t *offsets, int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                         int32_t *num_invalid, char *ws, hipStream_t s, int rounds = 1,
                         size_t round_bytes = 0);

// Quantisation modes; the values are those of ep_quant_t.
constexpr int kQuantBf16 = 0;
constexpr int kQuantFp8G128 = 1;
constexpr int kQuantFp8Token = 2;
constexpr int kQuantInt8Token = 3;
constexpr int kQuantMxE4M3 = 4;
constexpr int kQuantMxE5M2 = 5;
constexpr int kQuantMxE2M1 = 6;

hipError_t launch_dispatch(const LayoutPlan &p, const uint16_t *x, int H, const int32_t *topk_idx,
                           const int32_t *offsets, bool padded, int cap_or_rows, int quant,
                           void *recv_x, void *recv_scales, int32_t *slot, int32_t *recv_src,
                           int32_t *num_dropped, char *ws, hipStream_t s);

// The one-launch low-latency dispatch (padded rows, ranks found in the
// kernel): each block scans the entries before its token, so it is built for
// small batches.
constexpr int kLlMaxEntries = 4096;   // T*K
constexpr int kLlMaxTopk = 64;        // one lane per (t,k)
bool ll_dispatch_fits(int T, int K, int H, int quant);
hipError_t launch_ll_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx, int K,
                              int E, int cap, int quant, void *recv_x, void *recv_scales,
                              int32_t *slot, int32_t *recv_src, int32_t *recv_count,
                              int32_t *num_dropped, int32_t *num_invalid, hipStream_t s);

hipError_t launch_combine(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                          const float *w, int T, int K, uint16_t *out, hipStream_t s);

// The combine with fp32 output rows: the receiving rank's partial sums.
hipError_t launch_combine_partial(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                                  const float *w, int S, int K, float *partial, hipStream_t s);

// The sender pack (rank layout + rank_pack_kernel) and the sender's sum of
// the partials over ranks (ep_rank.hip).
hipError_t launch_rank_pack(const RankPlan &rp, const uint16_t *x, int H, const int32_t *topk_idx,
                            const float *w, int E, int R, int max_rows, int32_t *tokens_per_rank,
                            int32_t *rank_offsets, uint16_t *send_x, int32_t *send_src,
                            int32_t *send_idx, float *send_w, int32_t *pack_pos,
                            int32_t *num_dropped, char *ws, hipStream_t s);
hipError_t launch_rank_sum(const float *partial, int rows, int H, const int32_t *pack_pos, int T,
                           int R, uint16_t *out, hipStream_t s);

hipError_t launch_ec_dispatch(const EcPlan &p, const uint16_t *x, int H,
                              const int32_t *token_indices, uint16_t *recv_x, int32_t *tok_off,
                              int32_t *tok_ent, int32_t *num_invalid, char *ws, hipStream_t s);

hipError_t launch_ec_combine(const uint16_t *y, const float *w, int E, int C, int H,
                             const int32_t *tok_off, const int32_t *tok_ent, int T,
                             uint16_t *out, hipStream_t s);

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// LDS bytes one block may take on the current device (cached per device).
int lds_limit();

}  // namespace ep
