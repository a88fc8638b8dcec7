"""Helpers for the GPU tests: host<->device copies of bit patterns, and
calls through the C ABI with caller-owned buffers."""
import numpy as np
import torch

import combine_get_dispatch_04_amd._native as N
import tolerance as _tol

DEV = "cuda"
SENT16 = 0x7BAD      # sentinel bf16 pattern for rows nobody should write
SENT8 = 0x5A


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint8:
        return torch.from_numpy(a).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def p(t):
    return None if t is None else t.data_ptr()


def layout(idx_d: torch.Tensor, E: int, R: int = 1, with_rank=True):
    T, K = idx_d.shape
    wsb = N.ep_workspace_bytes(T, K, E, R)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    out = dict(counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
               offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
               tokens_per_rank=torch.full((R,), -7, dtype=torch.int32, device=DEV) if with_rank else None,
               is_token_in_rank=torch.full((T, R), 9, dtype=torch.uint8, device=DEV) if with_rank else None,
               num_invalid=torch.full((1,), -7, dtype=torch.int32, device=DEV))
    N.ep_get_dispatch_layout(p(idx_d), T, K, E, R, p(out["counts"]), p(out["offsets"]),
                             p(out["tokens_per_rank"]), p(out["is_token_in_rank"]),
                             p(out["num_invalid"]), p(ws), wsb, stream())
    out["ws"] = ws
    return out


SENT_E8M0 = 0xEE     # an e8m0 code only for block maxima of 2^111 and above (not in the tests)


def quant_buffers(quant, rows, H, sentinel=True):
    """Receive payload and scale arrays of ep_quant_t `quant` (>= 1), filled
    with sentinels."""
    rb = H // 2 if quant == N.EP_QUANT_MXFP4_E2M1 else H
    recv = torch.full((rows, rb), SENT8 if sentinel else 0, dtype=torch.uint8, device=DEV)
    if quant == N.EP_QUANT_FP8_E4M3_G128:
        sc = torch.full((rows, H // 128), -1.0, dtype=torch.float32, device=DEV)
    elif quant in (N.EP_QUANT_FP8_E4M3_TOKEN, N.EP_QUANT_INT8_TOKEN):
        sc = torch.full((max(rows, 1),), -1.0, dtype=torch.float32, device=DEV)
    else:
        sc = torch.full((rows, H // 32), SENT_E8M0, dtype=torch.uint8, device=DEV)
    return recv, sc


def dispatch(x_d, idx_d, E, L, padded=False, cap_or_rows=None, fp8=False, sentinel=True, quant=None):
    T, H = x_d.shape
    K = idx_d.shape[1]
    if cap_or_rows is None:
        cap_or_rows = T * K
    rows = E * cap_or_rows if padded else cap_or_rows
    if quant is None:
        quant = N.EP_QUANT_FP8_E4M3_G128 if fp8 else N.EP_QUANT_BF16
    if quant != N.EP_QUANT_BF16:
        recv, sc = quant_buffers(quant, rows, H, sentinel)
    else:
        recv = torch.full((rows, H), SENT16 if sentinel else 0, dtype=torch.int16,
                          device=DEV).view(torch.bfloat16)
        sc = None
    slot = torch.full((T, K), -9, dtype=torch.int32, device=DEV)
    src = torch.full((max(rows, 1),), -2, dtype=torch.int32, device=DEV)
    nd = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    N.ep_dispatch(p(x_d), T, H, p(idx_d), K, E, p(L["offsets"]), int(padded), cap_or_rows,
                  int(quant), p(recv), p(sc), p(slot), p(src), p(nd), p(L["ws"]), L["ws"].numel(),
                  stream())
    return recv, sc, slot, src, nd


def combine(y_d, slot_d, w_d):
    T, K = slot_d.shape
    H = y_d.shape[1]
    out = torch.full((T, H), SENT16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    N.ep_combine(p(y_d), y_d.shape[0], H, p(slot_d), p(w_d), T, K, p(out), stream())
    return out


def ec_dispatch(x_d, ti_d):
    T, H = x_d.shape
    E, C = ti_d.shape
    wsb = N.ep_ec_workspace_bytes(T, E, C)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    recv = torch.full((E, C, H), SENT16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    off = torch.full((T + 1,), -7, dtype=torch.int32, device=DEV)
    ent = torch.full((E * C,), -2, dtype=torch.int32, device=DEV)
    ninv = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    N.ep_dispatch_expert_choice(p(x_d), T, H, p(ti_d), E, C, p(recv), p(off), p(ent), p(ninv),
                                p(ws), wsb, stream())
    return recv, off, ent, ninv


def ec_combine(y_d, w_d, off_d, ent_d, T):
    E, C, H = y_d.shape
    out = torch.full((T, H), SENT16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    N.ep_combine_expert_choice(p(y_d), p(w_d), E, C, H, p(off_d), p(ent_d), T, p(out), stream())
    return out


# the combine tolerance (NaN-proof; see tests/tolerance.py)
bf16_f64 = _tol.bf16_f64
assert_combine_close = _tol.assert_combine_close
assert_f32_close = _tol.assert_f32_close


# ---------------------------------------------------------------- one rank's share
def pack_by_rank(x_d, idx_d, w_d, E, R, max_rows=None):
    """ep_pack_by_rank with sentinel-filled outputs."""
    T, H = x_d.shape
    K = idx_d.shape[1]
    if max_rows is None:
        max_rows = T * min(K, R)
    wsb = N.ep_pack_workspace_bytes(T, K, E, R)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    o = dict(tokens_per_rank=torch.full((R,), -7, dtype=torch.int32, device=DEV),
             rank_offsets=torch.full((R + 1,), -7, dtype=torch.int32, device=DEV),
             send_x=torch.full((max(max_rows, 1), H), SENT16, dtype=torch.int16,
                               device=DEV).view(torch.bfloat16),
             send_src=torch.full((max(max_rows, 1),), -2, dtype=torch.int32, device=DEV),
             send_idx=torch.full((max(max_rows, 1), K), -3, dtype=torch.int32, device=DEV),
             send_w=torch.full((max(max_rows, 1), K), -5.0, dtype=torch.float32, device=DEV),
             pack_pos=torch.full((T, R), -9, dtype=torch.int32, device=DEV),
             num_dropped=torch.full((1,), -7, dtype=torch.int32, device=DEV))
    N.ep_pack_by_rank(p(x_d), T, H, p(idx_d), p(w_d), K, E, R, max_rows, p(o["tokens_per_rank"]),
                      p(o["rank_offsets"]), p(o["send_x"]), p(o["send_src"]), p(o["send_idx"]),
                      p(o["send_w"]), p(o["pack_pos"]), p(o["num_dropped"]), p(ws), wsb,
                      stream())
    o["ws"] = ws
    return o


def combine_partial(y_d, slot_d, w_d):
    S, K = slot_d.shape
    H = y_d.shape[1]
    part = torch.full((S, H), float("nan"), dtype=torch.float32, device=DEV)
    N.ep_combine_partial(p(y_d), y_d.shape[0], H, p(slot_d), p(w_d), S, K, p(part), stream())
    return part


def combine_ranks(part_d, pos_d):
    T, R = pos_d.shape
    H = part_d.shape[1]
    out = torch.full((T, H), SENT16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    N.ep_combine_ranks(p(part_d), part_d.shape[0], H, p(pos_d), T, R, p(out), stream())
    return out
