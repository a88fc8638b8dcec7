/*
 * ep.h -- C ABI of libep: MoE token dispatch/combine on one MI355X (gfx950).
 *
 * The operations follow two pages:
 *   [EPA] "DeepEP-Ascend" README: the "API Overview" table
 *         (get_dispatch_layout, dispatch, combine, low_latency_dispatch,
 *         low_latency_combine), the "Environment Variables" table
 *         (MOE_EXPERT_TOKEN_NUMS_TYPE: per-expert count or prefix sum;
 *         MOE_ENABLE_TOPK_NEG_ONE: a -1 in topk_idx means "not dispatched")
 *         and the "Quantization Modes in Normal Dispatch" table
 *         (float8_e4m3fn payload with float32 scales).
 *   [ECR] "[Feature Request] Support Expert-Choice Routing via Native
 *         Expert-Centric API ([num_experts, capacity])", "Proposed
 *         Solutions", Solution 1: token_indices [num_experts, capacity]
 *         int32 picked by each expert, plus per-entry expert weights.
 *
 * Conventions for every entry point
 *   - Notation: T tokens, H hidden channels, E experts, K = num_topk,
 *     R ranks (experts split into R equal contiguous blocks), C capacity,
 *     N = number of valid (t,k) slots.
 *   - bf16 values travel as uint16_t bit patterns, fp8 e4m3 as uint8_t codes.
 *   - Every array pointer is DEVICE memory, row-major, owned by the caller;
 *     libep allocates nothing and keeps no state between calls (beyond a
 *     cache of each device's shared-memory size per block).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and runs asynchronously.  Outputs are valid once the stream reaches
 *     the end of the call's work.
 *   - Argument errors are found on the host before anything is enqueued and
 *     returned synchronously (EP_ERR_INVALID_ARG / EP_ERR_UNSUPPORTED /
 *     EP_ERR_WORKSPACE).  A failed launch returns EP_ERR_HIP, as does a
 *     grid beyond the launch limit (about 16.7 million tokens or
 *     expert-choice entries per call: T times up to 256 threads must fit in
 *     32 bits), with nothing enqueued.  Bad DATA
 *     (an index out of range, a capacity overflow) never fails a call: it
 *     is counted in num_invalid / num_dropped and skipped, so every output
 *     stays defined.
 *   - Array base pointers must be 16-byte aligned; `ws` 256-byte aligned.
 *   - H % 8 == 0 (rows move in 16-byte pieces) and H <= 2^24
 *     (EP_ERR_UNSUPPORTED beyond: a row's byte count stays 32-bit); T*K,
 *     E*C and receive row counts < 2^31.  Byte offsets into buffers are
 *     64-bit, so buffers may exceed 4 GiB.
 *   - Results are deterministic: the same inputs give the same bytes.
 */
#ifndef EP_H
#define EP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes, receive layouts and quantisation modes are passed as
 * int32_t, with the named values below.  (Not as the enum types: a C++
 * function may not even read an enum parameter that holds a value outside
 * its enumerators' range, and every value a caller passes is checked.) */
typedef int32_t ep_status_t;
enum {
    EP_OK = 0,
    EP_ERR_INVALID_ARG = 1,   /* a size, pointer or alignment is wrong */
    EP_ERR_UNSUPPORTED = 2,   /* a valid request outside what is built (e.g. E > 4096) */
    EP_ERR_WORKSPACE = 3,     /* ws is NULL, misaligned or smaller than required */
    EP_ERR_HIP = 4            /* the HIP runtime reported a launch error */
};

typedef int32_t ep_recv_layout_t;
enum {
    EP_LAYOUT_CONTIGUOUS = 0, /* expert blocks back to back: expert e's rows start at offsets[e] */
    EP_LAYOUT_PADDED = 1      /* [E, cap] rows: expert e's rows start at e*cap (low-latency form) */
};

typedef int32_t ep_quant_t;
enum {
    EP_QUANT_BF16 = 0,           /* rows copied as bf16 */
    EP_QUANT_FP8_E4M3_G128 = 1,  /* e4m3 codes + one fp32 scale per 128 channels */
    EP_QUANT_FP8_E4M3_TOKEN = 2, /* e4m3 codes + one fp32 scale per token ("pertoken_fp8_e4m3") */
    EP_QUANT_INT8_TOKEN = 3,     /* int8 codes + one fp32 scale per token ("int8") */
    EP_QUANT_MXFP8_E4M3 = 4,     /* e4m3 codes + one e8m0 scale per 32 channels ("mx_fp8_e4m3") */
    EP_QUANT_MXFP8_E5M2 = 5,     /* e5m2 codes + one e8m0 scale per 32 channels ("mx_fp8_e5m2") */
    EP_QUANT_MXFP4_E2M1 = 6      /* e2m1 codes, 2 per byte, + e8m0 per 32 ("mx_fp4_e2m1") */
};

/* Human-readable name of a status code (static string). */
const char *ep_status_string(ep_status_t status);

/* Bytes of device workspace that ep_get_dispatch_layout + ep_dispatch need
 * for these sizes (0 is never returned for valid sizes). */
size_t ep_workspace_bytes(int T, int K, int E, int R);

/* Bytes of device workspace that ep_dispatch_expert_choice needs. */
size_t ep_ec_workspace_bytes(int T, int E, int C);

/*
 * ep_get_dispatch_layout -- [EPA] API Overview, get_dispatch_layout; the
 * count and prefix-sum forms of [EPA] Environment Variables.
 *
 *   topk_idx          [T, K] int32 in.  -1 = not dispatched; any other value
 *                     outside [0, E) is invalid (counted, then ignored).
 *   counts            [E] int32 out: valid (t,k) per expert.
 *   offsets           [E+1] int32 out: exclusive prefix sum, offsets[E] = N.
 *   tokens_per_rank   [R] int32 out or NULL: tokens with >= 1 valid slot on
 *                     rank r (rank r owns experts [r*E/R, (r+1)*E/R)).
 *   is_token_in_rank  [T, R] uint8 out or NULL: 1 if token t has >= 1 valid
 *                     slot on rank r, else 0.
 *   num_invalid       [1] int32 out: entries that are neither -1 nor in [0,E).
 *   ws, ws_bytes      workspace of >= ep_workspace_bytes(T, K, E, R) bytes.
 *                     It carries per-chunk tables to the following
 *                     ep_dispatch, which must get the same ws, topk_idx, T,
 *                     K and E on the same stream with no other use of ws in
 *                     between.
 * Constraints: T >= 0, K >= 1 (no other limit: T*K < 2^31), 1 <= E <= 4096,
 * 1 <= R <= 1024, E % R == 0.
 */
ep_status_t ep_get_dispatch_layout(const int32_t *topk_idx, int T, int K, int E, int R,
                                   int32_t *counts, int32_t *offsets,
                                   int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                                   int32_t *num_invalid, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * ep_get_dispatch_layout_rounds -- the layout of a long prefill cut into
 * rounds of at most `round_tokens` tokens ([V4] custom_params:
 * moe_chunk_max_len, the token count of one MoE round), every round at once:
 * two launches in all instead of two per round.  Round r covers tokens
 * [r*round_tokens, min(T, (r+1)*round_tokens)); nr = ceil(T / round_tokens)
 * rounds.  Each round's outputs equal those of ep_get_dispatch_layout on
 * that round's rows of topk_idx alone, laid out round after round:
 *   counts            [nr, E] int32 out.
 *   offsets           [nr, E+1] int32 out (round-local: each starts at 0).
 *   tokens_per_rank   [nr, R] int32 out or NULL.
 *   is_token_in_rank  [T, R] uint8 out or NULL (token rows, as one call).
 *   num_invalid       [nr] int32 out.
 *   ws, ws_bytes      >= ep_workspace_bytes_rounds(T, K, E, R, round_tokens).
 *                     Round r's tables start S*r bytes into ws, where
 *                     S = ep_workspace_bytes(round_tokens, K, E, R); the
 *                     round's ep_dispatch takes that slice (ws + S*r, and
 *                     ws_bytes = ep_workspace_bytes(T_r, K, E, R) for the
 *                     round's T_r tokens), with x, topk_idx and offsets of
 *                     the round, on the same stream.
 * Constraints: those of ep_get_dispatch_layout, and round_tokens >= 1.
 * Errors as ep_get_dispatch_layout.
 */
size_t ep_workspace_bytes_rounds(int T, int K, int E, int R, int round_tokens);
ep_status_t ep_get_dispatch_layout_rounds(const int32_t *topk_idx, int T, int K, int E, int R,
                                          int round_tokens, int32_t *counts, int32_t *offsets,
                                          int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                                          int32_t *num_invalid, void *ws, size_t ws_bytes,
                                          void *stream);

/*
 * ep_dispatch -- [EPA] API Overview, dispatch (contiguous receive buffer)
 * and low_latency_dispatch (per-expert capacity); [EPA] Quantization Modes
 * in Normal Dispatch (bf16; INT8 dynamic and scalar FP8 per token with
 * float32 scales; MXFP8 e4m3/e5m2 and MXFP4 e2m1 with float8_e8m0fnu scales
 * per 32 elements), plus e4m3 with a float32 scale per 128 channels.
 *
 * The receive row ("slot") of a valid (t,k) with expert e is found by a
 * stable counting sort: r = number of valid (t',k') before (t,k) in
 * row-major order with the same expert.
 *   EP_LAYOUT_CONTIGUOUS: slot = offsets[e] + r, kept if slot < rows
 *                         (rows = cap_or_max_rows; T*K always suffices).
 *   EP_LAYOUT_PADDED:     slot = e*cap + r, kept if r < cap
 *                         (cap = cap_or_max_rows; rows = E*cap).
 * Slots that are not kept are -1 and counted in num_dropped; padding and
 * invalid entries are -1 and not counted.  For each kept slot:
 *   EP_QUANT_BF16:          recv_x[slot, :] = x[t, :]  (bf16 bits, [rows, H])
 *   EP_QUANT_FP8_E4M3_G128: per token and 128-channel group g, with
 *                           a = max|x| over the group: s = a / 448 in fp32
 *                           (0 when a == 0), q = e4m3(x / s) rounded to
 *                           nearest even with fp32 division (all zero when
 *                           a == 0); recv_x[slot, :] = q (uint8 [rows, H]),
 *                           recv_scales[slot, g] = s (fp32 [rows, H/128]).
 *                           Needs H % 128 == 0.
 *   EP_QUANT_FP8_E4M3_TOKEN, EP_QUANT_INT8_TOKEN: the same with one group per
 *                           token: a = max|x| over the row, s = a / 448
 *                           (e4m3) or a / 127 (int8: q = x / s rounded to
 *                           nearest even, clamped to [-127, 127], stored as
 *                           two's complement bytes); recv_x uint8 [rows, H],
 *                           recv_scales fp32 [rows].  Any H: a row too long
 *                           for one block gets its max from a first kernel
 *                           (the workspace holds one float per token).
 *   EP_QUANT_MXFP8_E4M3, EP_QUANT_MXFP8_E5M2, EP_QUANT_MXFP4_E2M1: per token
 *                           and 32-channel block b, with a = max|x| over the
 *                           block: E = floor(log2(a)) - emax (emax = 8, 15,
 *                           2), clamped to [-127, 127], E = -127 when a == 0;
 *                           recv_scales[slot, b] = E + 127 (e8m0 code, uint8
 *                           [rows, H/32]); element = x * 2^-E (exact)
 *                           rounded to nearest even in the element format,
 *                           saturating at its largest finite value (448,
 *                           57344, 6).  recv_x is uint8 [rows, H] (fp8) or
 *                           [rows, H/2] (e2m1: channel 2i in the low nibble
 *                           of byte i, 2i+1 in the high nibble).  Needs
 *                           H % 32 == 0.
 *   x            [T, H] bf16 in; finite for the quantised modes (an infinity
 *                or NaN gives unspecified codes and scales in its group).
 *   topk_idx     [T, K] int32 in (the array given to ep_get_dispatch_layout).
 *   offsets      [E+1] int32 in, from ep_get_dispatch_layout.
 *   recv_x       [rows, row bytes] out (row bytes: 2H bf16, H for the 8-bit
 *                codes, H/2 for e2m1); rows that receive no token are not
 *                written.
 *   recv_scales  out, as given for each mode above (NULL for bf16): fp32
 *                aligned to 4 bytes, e8m0 codes any alignment.
 *   slot         [T, K] int32 out: the handle for ep_combine.
 *   recv_src     [rows] int32 out or NULL: recv_src[slot] = t for kept slots;
 *                other entries are not written.
 *   num_dropped  [1] int32 out.
 *   ws, ws_bytes the workspace just used by ep_get_dispatch_layout.
 */
ep_status_t ep_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx, int K, int E,
                        const int32_t *offsets, ep_recv_layout_t layout, int cap_or_max_rows,
                        ep_quant_t quant, void *recv_x, void *recv_scales,
                        int32_t *slot, int32_t *recv_src, int32_t *num_dropped,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * ep_low_latency_dispatch -- [EPA] API Overview, low_latency_dispatch(x,
 * topk_idx, num_max_dispatch_tokens_per_rank, num_experts): the decode-phase
 * dispatch into the capacity-padded buffer, in one launch, with no layout
 * call and no workspace.  slot, recv_x, recv_scales, recv_src and
 * num_dropped are exactly those of ep_get_dispatch_layout followed by
 * ep_dispatch with EP_LAYOUT_PADDED and cap_or_max_rows = cap (same
 * arguments, same quantisation modes); in addition
 *   recv_count   [E] int32 out: min(cap, valid (t,k) with expert e), the
 *                rows of expert e that hold a token (rows e*cap ..
 *                e*cap + recv_count[e] - 1).
 *   num_invalid  [1] int32 out: entries neither -1 nor in [0, E).
 * Each block ranks its own token's entries by counting equal experts among
 * the entries before them, so the work grows as (T*K)^2: built for decode
 * batches.  Limits (EP_ERR_UNSUPPORTED beyond them; the layout + dispatch
 * pair has none of these): T*K <= 4096, K <= 64, and for the per-token
 * modes a row that one block holds (H <= 8192 when H/8 is even, else
 * H <= 4096).  Other constraints as ep_dispatch, with 1 <= E <= 4096,
 * cap >= 0 and E*cap < 2^31.
 */
ep_status_t ep_low_latency_dispatch(const uint16_t *x, int T, int H, const int32_t *topk_idx,
                                    int K, int E, int cap, ep_quant_t quant, void *recv_x,
                                    void *recv_scales, int32_t *slot, int32_t *recv_src,
                                    int32_t *recv_count, int32_t *num_dropped,
                                    int32_t *num_invalid, void *stream);

/*
 * ep_layout_dispatch_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): ep_get_dispatch_layout followed by ep_dispatch in one
 * call, with no workspace argument.  The per-chunk tables and per-entry
 * ranks that the pair keeps in `ws` live instead in a device array inside
 * the library, EP_NOALLOC_SCRATCH_BYTES per device, held from the library's
 * first call on that device until the process ends.  Every output (counts,
 * offsets, tokens_per_rank, is_token_in_rank, num_invalid, recv_x,
 * recv_scales, slot, recv_src, num_dropped) is exactly the pair's for the
 * same arguments, which follow the two calls' rules (R as in
 * ep_get_dispatch_layout).
 *   - Nothing is allocated: no hipMalloc, no workspace, no allocating
 *     library routine.  The caller still provides every input and output.
 *   - Sizes whose tables exceed the array (ep_workspace_bytes(T, K, E, R) >
 *     EP_NOALLOC_SCRATCH_BYTES, e.g. T*K beyond about 1.9 million entries)
 *     return EP_ERR_UNSUPPORTED with nothing enqueued: use the pair.
 *   - All calls on one device share its array, and each call's layout
 *     rewrites every entry the dispatch then reads, so nothing needs
 *     clearing; but two calls whose work overlaps on one device (on
 *     different streams, or from different threads) race on the array and
 *     give undefined results.  Serialise them.
 *   - EP_ERR_HIP also when the runtime cannot give the array's address on
 *     the stream's device.
 */
#define EP_NOALLOC_SCRATCH_BYTES (8u << 20)
ep_status_t ep_layout_dispatch_noalloc(const uint16_t *x, int T, int H, const int32_t *topk_idx,
                                       int K, int E, int R, int32_t *counts, int32_t *offsets,
                                       int32_t *tokens_per_rank, uint8_t *is_token_in_rank,
                                       int32_t *num_invalid, ep_recv_layout_t layout,
                                       int cap_or_max_rows, ep_quant_t quant, void *recv_x,
                                       void *recv_scales, int32_t *slot, int32_t *recv_src,
                                       int32_t *num_dropped, void *stream);

/*
 * ep_combine -- [EPA] API Overview, combine (reduce through the dispatch
 * handle) and low_latency_combine (also takes topk_weights).
 *   out[t, :] = bf16( sum over k with slot[t,k] >= 0 of w[t,k] * y[slot[t,k], :] )
 * summed in fp32, rounded to nearest even; a token with no kept slot gives +0.
 *   y             [y_rows, H] bf16 in, rows indexed like recv_x.
 *   slot          [T, K] int32 in, from ep_dispatch; entries outside
 *                 [0, y_rows) are skipped like -1 (a malformed handle cannot
 *                 make the kernel read outside y).
 *   topk_weights  [T, K] fp32 in, or NULL for unit weights (a plain sum).
 *   out           [T, H] bf16 out; must not overlap y.
 */
ep_status_t ep_combine(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                       const float *topk_weights, int T, int K, uint16_t *out, void *stream);

/*
 * ep_dispatch_expert_choice -- [ECR] Solution 1.
 *   recv_x[e, c, :] = x[token_indices[e, c], :] for entries in [0, T);
 *   -1 entries are empty and leave their row unwritten; other values are
 *   invalid (counted in num_invalid, row unwritten).  Duplicates are allowed.
 * It also builds the inverse map kept as the handle for combine:
 *   tok_off [T+1] int32 out, tok_ent [E*C] int32 out: token t's flat entries
 *   j = e*C + c, ascending, are tok_ent[tok_off[t] .. tok_off[t+1]);
 *   tok_off[T] = number of valid entries; tok_ent beyond it is not written.
 *   x             [T, H] bf16 in.
 *   token_indices [E, C] int32 in.
 *   recv_x        [E, C, H] bf16 out.
 *   num_invalid   [1] int32 out.
 *   ws, ws_bytes  workspace of >= ep_ec_workspace_bytes(T, E, C) bytes.
 * No limit on how many experts pick one token.
 */
ep_status_t ep_dispatch_expert_choice(const uint16_t *x, int T, int H,
                                      const int32_t *token_indices, int E, int C,
                                      uint16_t *recv_x, int32_t *tok_off, int32_t *tok_ent,
                                      int32_t *num_invalid, void *ws, size_t ws_bytes,
                                      void *stream);

/*
 * ep_combine_expert_choice -- [ECR] Solution 1 (the weights passed with the
 * expert-centric indices).
 *   out[t, :] = bf16( sum over j in tok_ent[tok_off[t] .. tok_off[t+1]) of
 *                     weights[j] * y[j, :] ), fp32 sums, nearest-even rounding;
 *   tokens that no expert picked give +0.
 *   y        [E, C, H] bf16 in.     weights [E, C] fp32 in.
 *   tok_off, tok_ent                from ep_dispatch_expert_choice; a token
 *            whose range is not inside [0, E*C], and entries outside
 *            [0, E*C), contribute nothing.
 *   out      [T, H] bf16 out; must not overlap y.
 */
ep_status_t ep_combine_expert_choice(const uint16_t *y, const float *weights, int E, int C, int H,
                                     const int32_t *tok_off, const int32_t *tok_ent, int T,
                                     uint16_t *out, void *stream);

/*
 * One rank's share of the expert-parallel exchange -- [EPA] API Overview:
 * get_dispatch_layout returns num_tokens_per_rank and is_token_in_rank,
 * dispatch sends each token to the ranks that hold its experts ("tokens to
 * expert ranks"), and combine reduces what comes back.  Rank r owns experts
 * [r*E/R, (r+1)*E/R).  The exchange between ranks is not part of libep:
 * what a sender packs for rank r is what rank r receives from it, and the
 * partial sums rank r returns are what the sender adds.
 *
 *   sender:    ep_pack_by_rank
 *   receiver:  the rows it received from the source ranks, concatenated in
 *              source-rank order, scattered into its E/R experts by
 *              ep_get_dispatch_layout + ep_dispatch with topk_idx = the
 *              received send_idx rows and E/R experts: the stable scatter,
 *              so an expert's rows are in (source rank, source token, k)
 *              order; then, after the experts, ep_combine_partial with the
 *              received send_w rows as weights
 *   sender:    ep_combine_ranks over the returned partial rows
 */

/* Bytes of device workspace that ep_pack_by_rank needs. */
size_t ep_pack_workspace_bytes(int T, int K, int E, int R);

/*
 * ep_pack_by_rank -- the sender's rows, grouped by destination rank: token t
 * is sent once to each rank r that holds at least one of its valid entries
 * (is_token_in_rank[t, r] of ep_get_dispatch_layout), as one row of x with
 * the token's K entries rewritten for r.  Rows are ordered by rank, then by
 * token (a stable counting sort keyed by (rank, token)):
 *   tokens_per_rank [R] int32 out: tokens sent to rank r.
 *   rank_offsets    [R+1] int32 out: exclusive prefix sum of tokens_per_rank;
 *                   rank r's rows start at rank_offsets[r].
 *   row of (t, r):  p = rank_offsets[r] + number of tokens t' < t sent to r;
 *                   kept if p < max_rows (T * min(K, R) always suffices),
 *                   else counted in num_dropped.  For each kept row:
 *   send_x   [max_rows, H] bf16 out: send_x[p] = x[t].
 *   send_src [max_rows] int32 out: t.
 *   send_idx [max_rows, K] int32 out: for each k, topk_idx[t,k] - r*E/R
 *            (the local expert id) if entry k is valid and on rank r, else -1.
 *   send_w   [max_rows, K] fp32 out or NULL: topk_weights[t,k] (1 when
 *            topk_weights is NULL) where send_idx >= 0, else 0.
 *   pack_pos [T, R] int32 out: p for kept (t, r) rows, -1 otherwise (the
 *            handle for ep_combine_ranks).
 *   num_dropped [1] int32 out.
 * Rows p >= rank_offsets[R] are not written.  Invalid entries (neither -1
 * nor in [0, E)) are ignored like -1.
 *   ws, ws_bytes  workspace of >= ep_pack_workspace_bytes(T, K, E, R) bytes.
 * Constraints: those of ep_get_dispatch_layout (1 <= R <= 1024, E % R == 0),
 * H % 8 == 0, max_rows >= 0, T*R and max_rows*K < 2^31.
 */
ep_status_t ep_pack_by_rank(const uint16_t *x, int T, int H, const int32_t *topk_idx,
                            const float *topk_weights, int K, int E, int R, int max_rows,
                            int32_t *tokens_per_rank, int32_t *rank_offsets, uint16_t *send_x,
                            int32_t *send_src, int32_t *send_idx, float *send_w,
                            int32_t *pack_pos, int32_t *num_dropped, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * ep_combine_partial -- the receiving rank's combine: ep_combine with fp32
 * output rows, the partial sums that go back to the sender.
 *   partial[p, :] = sum over k with slot[p,k] in [0, y_rows) of
 *                   weights[p,k] * y[slot[p,k], :]
 * in fp32 (a row with no kept slot gives +0).
 *   y        [y_rows, H] bf16 in.   slot [S, K] int32 in (from ep_dispatch).
 *   weights  [S, K] fp32 in (the received send_w), or NULL for unit weights.
 *   partial  [S, H] fp32 out, 16-byte aligned; must not overlap y.
 */
ep_status_t ep_combine_partial(const uint16_t *y, int y_rows, int H, const int32_t *slot,
                               const float *weights, int S, int K, float *partial, void *stream);

/*
 * ep_combine_ranks -- the sender's sum after the reverse exchange:
 *   out[t, :] = bf16( sum over r = 0 .. R-1, in that order, with
 *                     pack_pos[t, r] in [0, rows), of partial[pack_pos[t,r], :] )
 * with fp32 adds, rounded once to nearest even; a token no rank received
 * gives +0.
 *   partial  [rows, H] fp32 in: the rows the receivers returned, at the
 *            positions their tokens had in send_x.
 *   pack_pos [T, R] int32 in (from ep_pack_by_rank).
 *   out      [T, H] bf16 out; must not overlap partial.
 * Constraints: 1 <= R <= 1024, H % 8 == 0, T*R < 2^31.
 */
ep_status_t ep_combine_ranks(const float *partial, int rows, int H, const int32_t *pack_pos,
                             int T, int R, uint16_t *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EP_H */
