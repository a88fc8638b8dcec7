"""Torch-tensor front end over the libep C ABI.

Mirrors the Buffer methods of the "DeepEP-Ascend" README ("API Overview":
get_dispatch_layout, dispatch, combine, low_latency_dispatch /
low_latency_combine) and the expert-centric calls asked for in "[Feature
Request] Support Expert-Choice Routing via Native Expert-Centric API"
(Solution 1: dispatch_expert_choice with token_indices [E, C] and weights).

torch only allocates device memory and supplies the current stream; every
step runs in the HIP kernels of libep.so.  Errors from the library raise
EpError (a ValueError).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import _native as N


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_device(dev: torch.device, **tensors):
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}")


def _out(out: Optional[torch.Tensor], shape, dev: torch.device) -> torch.Tensor:
    """A caller's output tensor, checked before the kernel writes shape[0] rows
    into it, or a new one."""
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must be {tuple(shape)}, got {tuple(out.shape)}")
    _same_device(dev, out=out)
    return out


@dataclass
class Layout:
    """Result of get_dispatch_layout.  The workspace carries per-chunk tables
    to the dispatch that follows and must not be reused before it."""
    num_tokens_per_rank: torch.Tensor          # [R] int32
    num_tokens_per_rdma_rank: None             # needs a node topology: not produced
    num_tokens_per_expert: torch.Tensor        # [E] int32 (count form)
    is_token_in_rank: torch.Tensor             # [T, R] uint8
    offsets: torch.Tensor                      # [E+1] int32 (prefix-sum form)
    num_invalid: torch.Tensor                  # [1] int32
    topk_idx: torch.Tensor
    num_experts: int
    num_ranks: int
    workspace: torch.Tensor


@dataclass
class Handle:
    """What combine needs from dispatch: the receive row of every (t, k)."""
    slot: torch.Tensor                         # [T, K] int32, -1 = not received
    recv_src: torch.Tensor                     # [rows] int32, source token of each written row
    num_dropped: torch.Tensor                  # [1] int32
    rows: int
    recv_layout: str
    cap: Optional[int]
    recv_count: Optional[torch.Tensor] = None  # [E] int32, rows each expert holds (low latency)
    num_invalid: Optional[torch.Tensor] = None  # [1] int32 (low latency)


@dataclass
class ExpertChoiceHandle:
    tok_off: torch.Tensor                      # [T+1] int32
    tok_ent: torch.Tensor                      # [E*C] int32
    weights: torch.Tensor                      # [E, C] float32
    num_invalid: torch.Tensor                  # [1] int32
    num_tokens: int


def get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int = 1) -> Layout:
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, K = topk_idx.shape
    E, R = int(num_experts), int(num_ranks)
    dev = topk_idx.device
    ws_bytes = N.ep_workspace_bytes(T, K, E, R)
    if ws_bytes == 0:
        raise N.EpError("ep_workspace_bytes", N.EP_ERR_INVALID_ARG)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    tpr = torch.empty(R, dtype=torch.int32, device=dev)
    itr = torch.empty((T, R), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        N.ep_get_dispatch_layout(_ptr(topk_idx), T, K, E, R, _ptr(counts), _ptr(offsets),
                                 _ptr(tpr), _ptr(itr), _ptr(ninv), _ptr(ws), ws_bytes,
                                 _stream(dev))
    return Layout(tpr, None, counts, itr, offsets, ninv, topk_idx, E, R, ws)


def get_dispatch_layout_rounds(topk_idx: torch.Tensor, num_experts: int, round_tokens: int,
                               num_ranks: int = 1) -> List[Layout]:
    """The layouts of rounds of at most `round_tokens` tokens ("DeepSeek-V4
    昇腾 NPU 推理部署实践", custom_params: moe_chunk_max_len), all from one
    call: round r's Layout equals get_dispatch_layout(topk_idx[r*rt:(r+1)*rt])
    and carries its own slice of the shared workspace for that round's
    dispatch."""
    _need(topk_idx, "topk_idx", torch.int32, 2)
    if round_tokens < 1:
        raise ValueError("round_tokens must be >= 1")
    T, K = topk_idx.shape
    E, R = int(num_experts), int(num_ranks)
    dev = topk_idx.device
    ws_bytes = N.ep_workspace_bytes_rounds(T, K, E, R, round_tokens)
    if ws_bytes == 0:
        raise N.EpError("ep_workspace_bytes_rounds", N.EP_ERR_INVALID_ARG)
    rt = min(round_tokens, T)
    nr = (T + rt - 1) // rt if T else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    counts = torch.empty((max(nr, 1), E), dtype=torch.int32, device=dev)
    offsets = torch.empty((max(nr, 1), E + 1), dtype=torch.int32, device=dev)
    tpr = torch.empty((max(nr, 1), R), dtype=torch.int32, device=dev)
    itr = torch.empty((T, R), dtype=torch.uint8, device=dev)
    ninv = torch.empty(max(nr, 1), dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        N.ep_get_dispatch_layout_rounds(_ptr(topk_idx), T, K, E, R, round_tokens, _ptr(counts),
                                        _ptr(offsets), _ptr(tpr), _ptr(itr), _ptr(ninv),
                                        _ptr(ws), ws_bytes, _stream(dev))
    stride = N.ep_workspace_bytes(rt, K, E, R) if nr else 0
    out = []
    for r in range(nr):
        t0, t1 = r * rt, min(T, (r + 1) * rt)
        b = N.ep_workspace_bytes(t1 - t0, K, E, R)
        out.append(Layout(tpr[r], None, counts[r], itr[t0:t1], offsets[r], ninv[r:r + 1],
                          topk_idx[t0:t1], E, R, ws[stride * r:stride * r + b]))
    return out


# quant name -> (ep_quant_t, receive dtype, H divisor of a receive row,
# scale shape: H -> (columns or 0 for one per row, dtype), or None)
_QUANT = {
    "bf16": (N.EP_QUANT_BF16, torch.bfloat16, 1, None),
    "fp8_e4m3_g128": (N.EP_QUANT_FP8_E4M3_G128, torch.float8_e4m3fn, 1,
                      lambda H: (H // 128, torch.float32)),
    "fp8_e4m3_token": (N.EP_QUANT_FP8_E4M3_TOKEN, torch.float8_e4m3fn, 1,
                       lambda H: (0, torch.float32)),
    "int8_token": (N.EP_QUANT_INT8_TOKEN, torch.int8, 1, lambda H: (0, torch.float32)),
    "mxfp8_e4m3": (N.EP_QUANT_MXFP8_E4M3, torch.float8_e4m3fn, 1, lambda H: (H // 32, torch.uint8)),
    "mxfp8_e5m2": (N.EP_QUANT_MXFP8_E5M2, torch.float8_e5m2, 1, lambda H: (H // 32, torch.uint8)),
    "mxfp4_e2m1": (N.EP_QUANT_MXFP4_E2M1, torch.uint8, 2, lambda H: (H // 32, torch.uint8)),
}
_QUANT_ALIASES = {"pertoken_fp8_e4m3": "fp8_e4m3_token", "int8": "int8_token",
                  "mx_fp8_e4m3": "mxfp8_e4m3", "mx_fp8_e5m2": "mxfp8_e5m2",
                  "mx_fp4_e2m1": "mxfp4_e2m1"}


def dispatch(x: torch.Tensor, layout: Layout, *, quant: str = "bf16",
             recv_layout: str = "contiguous", cap: Optional[int] = None,
             max_rows: Optional[int] = None):
    """-> (recv_x, recv_scales or None, Handle).

    recv_layout "contiguous": expert blocks back to back, `max_rows` rows
    (default T*K, always enough).  "padded": [E, cap] rows, the low-latency
    form.  quant (names of the DeepEP-Ascend quantisation modes in
    parentheses):
      "bf16"                                 recv bf16 [rows, H], no scales
      "fp8_e4m3_g128"                        e4m3 [rows, H] + fp32 [rows, H/128]
      "fp8_e4m3_token" ("pertoken_fp8_e4m3") e4m3 [rows, H] + fp32 [rows]
      "int8_token" ("int8")                  int8 [rows, H] + fp32 [rows]
      "mxfp8_e4m3" ("mx_fp8_e4m3")           e4m3 [rows, H] + e8m0 codes uint8 [rows, H/32]
      "mxfp8_e5m2" ("mx_fp8_e5m2")           e5m2 [rows, H] + e8m0 codes uint8 [rows, H/32]
      "mxfp4_e2m1" ("mx_fp4_e2m1")           uint8 [rows, H/2], two e2m1 codes per byte
                                             (low nibble first) + e8m0 uint8 [rows, H/32]"""
    _need(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    idx = layout.topk_idx
    if idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on the number of tokens")
    K, E = idx.shape[1], layout.num_experts
    quant = _QUANT_ALIASES.get(quant, quant)
    if quant not in _QUANT:
        raise ValueError(f"unknown quant mode {quant!r}")
    q, rdt, row_div, scale_shape = _QUANT[quant]
    if recv_layout == "contiguous":
        lay, arg = N.EP_LAYOUT_CONTIGUOUS, (T * K if max_rows is None else int(max_rows))
        rows = arg
    elif recv_layout == "padded":
        if cap is None:
            raise ValueError("padded layout needs cap")
        lay, arg = N.EP_LAYOUT_PADDED, int(cap)
        rows = E * arg
    else:
        raise ValueError(f"unknown receive layout {recv_layout!r}")
    dev = x.device
    _same_device(dev, topk_idx=idx, workspace=layout.workspace)
    recv = torch.empty((rows, H // row_div), dtype=rdt, device=dev)
    scales = None
    if scale_shape is not None:
        ncol, sdt = scale_shape(H)
        scales = torch.empty((rows, ncol) if ncol else (rows,), dtype=sdt, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        N.ep_dispatch(_ptr(x), T, H, _ptr(idx), K, E, _ptr(layout.offsets), lay, arg, q,
                      _ptr(recv), _ptr(scales), _ptr(slot), _ptr(src), _ptr(nd),
                      _ptr(layout.workspace), layout.workspace.numel(), _stream(dev))
    return recv, scales, Handle(slot, src, nd, rows, recv_layout, cap if lay else None)


def combine(y: torch.Tensor, handle: Handle, topk_weights: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[t] = bf16(sum_k w[t,k] * y[slot[t,k]]), fp32 sums; w = 1 if None."""
    _need(y, "y", torch.bfloat16, 2)
    T, K = handle.slot.shape
    H = y.shape[1]
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, 2)
        if tuple(topk_weights.shape) != (T, K):
            raise ValueError("topk_weights must be [T, K]")
    dev = y.device
    _same_device(dev, slot=handle.slot, topk_weights=topk_weights)
    out = _out(out, (T, H), dev)
    with torch.cuda.device(dev):
        N.ep_combine(_ptr(y), y.shape[0], H, _ptr(handle.slot), _ptr(topk_weights), T, K,
                     _ptr(out), _stream(dev))
    return out


def low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor,
                         num_max_dispatch_tokens_per_rank: int, num_experts: int, *,
                         quant: str = "fp8_e4m3_g128"):
    """The decode-phase call of "DeepEP-Ascend" README, API Overview
    (low_latency_dispatch(x, topk_idx, num_max_dispatch_tokens_per_rank,
    num_experts)): one launch, no layout call, into the capacity-padded buffer
    of num_max_dispatch_tokens_per_rank rows per expert.  Quantised by default
    (e4m3 with one fp32 scale per 128 channels); quant="bf16" turns it off.
    The same slots, codes and scales as get_dispatch_layout + dispatch with
    recv_layout="padded"; built for decode batches (T*K <= 4096, K <= 64),
    beyond which the library reports the request as unsupported and that pair
    is the call to use.
    -> (recv_x [E, cap, H or H/2], recv_scales [E, cap, ...] or None, Handle);
    the shapes are views of the flat receive rows, and handle.recv_count [E]
    holds the rows each expert received (at most cap)."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, H = x.shape
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on the number of tokens")
    K = topk_idx.shape[1]
    E, cap = int(num_experts), int(num_max_dispatch_tokens_per_rank)
    quant = _QUANT_ALIASES.get(quant, quant)
    if quant not in _QUANT:
        raise ValueError(f"unknown quant mode {quant!r}")
    q, rdt, row_div, scale_shape = _QUANT[quant]
    if E < 1 or cap < 0:
        raise ValueError("num_experts must be >= 1 and the capacity >= 0")
    rows = E * cap
    dev = x.device
    _same_device(dev, topk_idx=topk_idx)
    recv = torch.empty((rows, H // row_div), dtype=rdt, device=dev)
    scales = None
    if scale_shape is not None:
        ncol, sdt = scale_shape(H)
        scales = torch.empty((rows, ncol) if ncol else (rows,), dtype=sdt, device=dev)
    slot = torch.empty((T, K), dtype=torch.int32, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        N.ep_low_latency_dispatch(_ptr(x), T, H, _ptr(topk_idx), K, E, cap, q, _ptr(recv),
                                  _ptr(scales), _ptr(slot), _ptr(src), _ptr(cnt), _ptr(nd),
                                  _ptr(ninv), _stream(dev))
    recv = recv.view(E, cap, *recv.shape[1:])
    if scales is not None:
        scales = scales.view(E, cap, *scales.shape[1:])
    return recv, scales, Handle(slot, src, nd, rows, "padded", cap, cnt, ninv)


def low_latency_combine(y: torch.Tensor, topk_idx: torch.Tensor,
                        topk_weights: Optional[torch.Tensor], handle: Handle,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The decode-phase combine of "DeepEP-Ascend" README, API Overview
    (low_latency_combine(x, topk_idx, topk_weights, handle)): y holds the
    experts' bf16 rows in the receive layout, [E, cap, H] or [E*cap, H];
    out[t] = bf16(sum_k w[t,k] * y[slot[t,k]]) with fp32 sums.  topk_idx
    must be the one the handle came from (its shape is checked; the slots in
    the handle already encode it)."""
    if y.dim() == 3:
        _need(y, "y", torch.bfloat16, 3)
        y = y.view(-1, y.shape[-1])
    _need(topk_idx, "topk_idx", torch.int32, 2)
    if tuple(topk_idx.shape) != tuple(handle.slot.shape):
        raise ValueError("topk_idx does not match the handle")
    return combine(y, handle, topk_weights, out=out)


def dispatch_combine_chunked(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, *,
                             chunk: int, topk_weights: Optional[torch.Tensor] = None,
                             expert=None, quant: str = "bf16", num_ranks: int = 1,
                             keep_rounds: bool = False):
    """Long prefill in rounds of at most `chunk` tokens ("DeepSeek-V4 昇腾
    NPU 推理部署实践", custom_params: moe_chunk_max_len bounds the tokens an
    MoE layer handles at once, against running out of memory on long
    sequences).  One call lays out every round (get_dispatch_layout_rounds);
    each round then runs dispatch, `expert` and combine on its own slice of
    tokens, so a receive buffer holds chunk*K rows instead of T*K.  `expert(recv, scales, layout) -> y` maps the received rows to the
    bf16 rows combine reads (default: identity, bf16 only).  Results equal
    the unchunked call: a token's rows and their order do not depend on the
    other tokens of its round.  -> out [T, H], plus the per-round (layout,
    handle) pairs when keep_rounds is set."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    if expert is None and quant != "bf16":
        raise ValueError("a quantised dispatch needs an expert that returns bf16 rows")
    T = x.shape[0]
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on the number of tokens")
    out = torch.empty_like(x)
    rounds = []
    for r, L in enumerate(get_dispatch_layout_rounds(topk_idx, num_experts, chunk, num_ranks)):
        t0 = r * min(chunk, T)
        t1 = t0 + L.topk_idx.shape[0]
        recv, scales, h = dispatch(x[t0:t1], L, quant=quant)
        y = recv if expert is None else expert(recv, scales, L)
        combine(y, h, None if topk_weights is None else topk_weights[t0:t1], out=out[t0:t1])
        if keep_rounds:
            rounds.append((L, h))
    return (out, rounds) if keep_rounds else out


def dispatch_expert_choice(x: torch.Tensor, token_indices: torch.Tensor, weights: torch.Tensor):
    """-> (recv_x [E, C, H], ExpertChoiceHandle).  The weights are kept in the
    handle and applied by combine_expert_choice."""
    _need(x, "x", torch.bfloat16, 2)
    _need(token_indices, "token_indices", torch.int32, 2)
    _need(weights, "weights", torch.float32, 2)
    T, H = x.shape
    E, C = token_indices.shape
    if tuple(weights.shape) != (E, C):
        raise ValueError("weights must be [E, C] like token_indices")
    dev = x.device
    _same_device(dev, token_indices=token_indices, weights=weights)
    ws_bytes = N.ep_ec_workspace_bytes(T, E, C)
    if ws_bytes == 0:
        raise N.EpError("ep_ec_workspace_bytes", N.EP_ERR_INVALID_ARG)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    recv = torch.empty((E, C, H), dtype=torch.bfloat16, device=dev)
    off = torch.empty(T + 1, dtype=torch.int32, device=dev)
    ent = torch.empty(E * C, dtype=torch.int32, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        N.ep_dispatch_expert_choice(_ptr(x), T, H, _ptr(token_indices), E, C, _ptr(recv),
                                    _ptr(off), _ptr(ent), _ptr(ninv), _ptr(ws), ws_bytes,
                                    _stream(dev))
    return recv, ExpertChoiceHandle(off, ent, weights, ninv, T)


def combine_expert_choice(y: torch.Tensor, handle: ExpertChoiceHandle,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(y, "y", torch.bfloat16, 3)
    E, C, H = y.shape
    T = handle.num_tokens
    if tuple(handle.weights.shape) != (E, C):
        raise ValueError(f"y is [{E}, {C}, H] but the handle's weights are "
                         f"{tuple(handle.weights.shape)}")
    dev = y.device
    _same_device(dev, weights=handle.weights, tok_off=handle.tok_off, tok_ent=handle.tok_ent)
    out = _out(out, (T, H), dev)
    with torch.cuda.device(dev):
        N.ep_combine_expert_choice(_ptr(y), _ptr(handle.weights), E, C, H, _ptr(handle.tok_off),
                                   _ptr(handle.tok_ent), T, _ptr(out), _stream(dev))
    return out


# ---------------------------------------------------------------- one rank's share
@dataclass
class RankPack:
    """What the sender packs ("DeepEP-Ascend" README, API Overview: the
    dispatch sends each token to the ranks of its experts): rows grouped by
    destination rank, each token once per rank that holds one of its
    experts, with that rank's local expert ids."""
    num_tokens_per_rank: torch.Tensor          # [R] int32
    rank_offsets: torch.Tensor                 # [R+1] int32: rank r's rows start here
    send_x: torch.Tensor                       # [rows, H] bf16
    send_src: torch.Tensor                     # [rows] int32: source token
    send_idx: torch.Tensor                     # [rows, K] int32: local expert ids, -1 elsewhere
    send_w: torch.Tensor                       # [rows, K] float32: weights, 0 where send_idx is -1
    pack_pos: torch.Tensor                     # [T, R] int32: row of (t, r) or -1
    num_dropped: torch.Tensor                  # [1] int32
    num_ranks: int
    experts_per_rank: int


def pack_by_rank(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                 topk_weights: Optional[torch.Tensor] = None,
                 max_rows: Optional[int] = None) -> RankPack:
    """The sender's rows for R ranks (rank r owns experts [r E/R, (r+1) E/R)):
    rows ordered by rank, then token.  `max_rows` defaults to T * min(K, R),
    always enough; rows beyond it are dropped and counted."""
    _need(x, "x", torch.bfloat16, 2)
    _need(topk_idx, "topk_idx", torch.int32, 2)
    T, H = x.shape
    if topk_idx.shape[0] != T:
        raise ValueError("x and topk_idx disagree on the number of tokens")
    K = topk_idx.shape[1]
    E, R = int(num_experts), int(num_ranks)
    if topk_weights is not None:
        _need(topk_weights, "topk_weights", torch.float32, 2)
        if tuple(topk_weights.shape) != (T, K):
            raise ValueError("topk_weights must be [T, K]")
    dev = x.device
    _same_device(dev, topk_idx=topk_idx, topk_weights=topk_weights)
    rows = T * min(K, R) if max_rows is None else int(max_rows)
    ws_bytes = N.ep_pack_workspace_bytes(T, K, E, R)
    if ws_bytes == 0:
        raise N.EpError("ep_pack_workspace_bytes", N.EP_ERR_INVALID_ARG)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    tpr = torch.empty(R, dtype=torch.int32, device=dev)
    off = torch.empty(R + 1, dtype=torch.int32, device=dev)
    sx = torch.empty((rows, H), dtype=torch.bfloat16, device=dev)
    src = torch.empty(rows, dtype=torch.int32, device=dev)
    sidx = torch.empty((rows, K), dtype=torch.int32, device=dev)
    sw = torch.empty((rows, K), dtype=torch.float32, device=dev)
    pos = torch.empty((T, R), dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    with torch.cuda.device(dev):
        N.ep_pack_by_rank(_ptr(x), T, H, _ptr(topk_idx), _ptr(topk_weights), K, E, R, rows,
                          _ptr(tpr), _ptr(off), _ptr(sx), _ptr(src), _ptr(sidx), _ptr(sw),
                          _ptr(pos), _ptr(nd), _ptr(ws), ws_bytes, _stream(dev))
    return RankPack(tpr, off, sx, src, sidx, sw, pos, nd, R, E // R)


def receive(recv_x: torch.Tensor, recv_idx: torch.Tensor, experts_per_rank: int, *,
            quant: str = "bf16", max_rows: Optional[int] = None):
    """The receiving rank's scatter of the rows it received (the blocks of
    its source ranks, concatenated in rank order) into its local experts:
    the layout and the stable scatter with the received local ids as
    topk_idx, so an expert's rows are in (source rank, source token, k)
    order.  -> (Layout, recv, recv_scales or None, Handle)."""
    layout = get_dispatch_layout(recv_idx, experts_per_rank)
    recv, scales, handle = dispatch(recv_x, layout, quant=quant, max_rows=max_rows)
    return layout, recv, scales, handle


def combine_partial(y: torch.Tensor, handle: Handle, weights: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The receiving rank's combine: per received row, sum_k w * y[slot] in
    fp32, kept in fp32 for the sender (the partial sums of the exchange)."""
    _need(y, "y", torch.bfloat16, 2)
    S, K = handle.slot.shape
    H = y.shape[1]
    if weights is not None:
        _need(weights, "weights", torch.float32, 2)
        if tuple(weights.shape) != (S, K):
            raise ValueError("weights must be [rows, K]")
    dev = y.device
    _same_device(dev, slot=handle.slot, weights=weights)
    if out is None:
        out = torch.empty((S, H), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, 2)
        if tuple(out.shape) != (S, H):
            raise ValueError(f"out must be {(S, H)}, got {tuple(out.shape)}")
        _same_device(dev, out=out)
    with torch.cuda.device(dev):
        N.ep_combine_partial(_ptr(y), y.shape[0], H, _ptr(handle.slot), _ptr(weights), S, K,
                             _ptr(out), _stream(dev))
    return out


def combine_ranks(partial: torch.Tensor, pack: RankPack,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The sender's sum of the partial rows the ranks returned (at the rows
    their tokens had in send_x), in rank order, rounded once to bf16."""
    _need(partial, "partial", torch.float32, 2)
    T, R = pack.pack_pos.shape
    H = partial.shape[1]
    dev = partial.device
    _same_device(dev, pack_pos=pack.pack_pos)
    out = _out(out, (T, H), dev)
    with torch.cuda.device(dev):
        N.ep_combine_ranks(_ptr(partial), partial.shape[0], H, _ptr(pack.pack_pos), T, R,
                           _ptr(out), _stream(dev))
    return out
