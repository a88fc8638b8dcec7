"""ctypes binding of libep.so: the C ABI of include/ep.h, same names.

Only argument marshalling happens here; every step runs in the HIP kernels.
Loading fails loudly if the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libep.so")

EP_OK, EP_ERR_INVALID_ARG, EP_ERR_UNSUPPORTED, EP_ERR_WORKSPACE, EP_ERR_HIP = range(5)
EP_LAYOUT_CONTIGUOUS, EP_LAYOUT_PADDED = 0, 1
(EP_QUANT_BF16, EP_QUANT_FP8_E4M3_G128, EP_QUANT_FP8_E4M3_TOKEN, EP_QUANT_INT8_TOKEN,
 EP_QUANT_MXFP8_E4M3, EP_QUANT_MXFP8_E5M2, EP_QUANT_MXFP4_E2M1) = range(7)

# name -> (restype, argtypes); every pointer is passed as an integer address
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_ST = ctypes.c_int
SIGNATURES = {
    "ep_status_string": (ctypes.c_char_p, [_ST]),
    "ep_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "ep_ec_workspace_bytes": (_SZ, [_I, _I, _I]),
    "ep_get_dispatch_layout": (_ST, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ep_workspace_bytes_rounds": (_SZ, [_I, _I, _I, _I, _I]),
    "ep_get_dispatch_layout_rounds": (_ST, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                            _P]),
    "ep_dispatch": (_ST, [_P, _I, _I, _P, _I, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "ep_low_latency_dispatch": (_ST, [_P, _I, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                      _P, _P]),
    "ep_combine": (_ST, [_P, _I, _I, _P, _P, _I, _I, _P, _P]),
    "ep_layout_dispatch_noalloc": (_ST, [_P, _I, _I, _P, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I,
                                         _I, _P, _P, _P, _P, _P, _P]),
    "ep_pack_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "ep_pack_by_rank": (_ST, [_P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                              _P, _SZ, _P]),
    "ep_combine_partial": (_ST, [_P, _I, _I, _P, _P, _I, _I, _P, _P]),
    "ep_combine_ranks": (_ST, [_P, _I, _I, _P, _I, _I, _P, _P]),
    "ep_dispatch_expert_choice": (_ST, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "ep_combine_expert_choice": (_ST, [_P, _P, _I, _I, _I, _P, _P, _I, _P, _P]),
}

_lib = None


class EpError(ValueError):
    """A libep call returned an error status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libep.so is not built ({LIB_PATH}); run "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().ep_status_string(status).decode()


def _check(fn: str, status: int) -> int:
    if status != EP_OK:
        raise EpError(fn, status)
    return status


def ep_workspace_bytes(T: int, K: int, E: int, R: int) -> int:
    return lib().ep_workspace_bytes(T, K, E, R)


def ep_ec_workspace_bytes(T: int, E: int, C: int) -> int:
    return lib().ep_ec_workspace_bytes(T, E, C)


def ep_get_dispatch_layout(topk_idx, T, K, E, R, counts, offsets, tokens_per_rank,
                           is_token_in_rank, num_invalid, ws, ws_bytes, stream, check=True):
    st = lib().ep_get_dispatch_layout(topk_idx, T, K, E, R, counts, offsets, tokens_per_rank,
                                      is_token_in_rank, num_invalid, ws, ws_bytes, stream)
    return _check("ep_get_dispatch_layout", st) if check else st


def ep_workspace_bytes_rounds(T: int, K: int, E: int, R: int, round_tokens: int) -> int:
    return lib().ep_workspace_bytes_rounds(T, K, E, R, round_tokens)


def ep_get_dispatch_layout_rounds(topk_idx, T, K, E, R, round_tokens, counts, offsets,
                                  tokens_per_rank, is_token_in_rank, num_invalid, ws, ws_bytes,
                                  stream, check=True):
    st = lib().ep_get_dispatch_layout_rounds(topk_idx, T, K, E, R, round_tokens, counts, offsets,
                                             tokens_per_rank, is_token_in_rank, num_invalid, ws,
                                             ws_bytes, stream)
    return _check("ep_get_dispatch_layout_rounds", st) if check else st


def ep_dispatch(x, T, H, topk_idx, K, E, offsets, layout, cap_or_max_rows, quant, recv_x,
                recv_scales, slot, recv_src, num_dropped, ws, ws_bytes, stream, check=True):
    st = lib().ep_dispatch(x, T, H, topk_idx, K, E, offsets, layout, cap_or_max_rows, quant,
                           recv_x, recv_scales, slot, recv_src, num_dropped, ws, ws_bytes, stream)
    return _check("ep_dispatch", st) if check else st


def ep_low_latency_dispatch(x, T, H, topk_idx, K, E, cap, quant, recv_x, recv_scales, slot,
                            recv_src, recv_count, num_dropped, num_invalid, stream, check=True):
    st = lib().ep_low_latency_dispatch(x, T, H, topk_idx, K, E, cap, quant, recv_x, recv_scales,
                                       slot, recv_src, recv_count, num_dropped, num_invalid,
                                       stream)
    return _check("ep_low_latency_dispatch", st) if check else st


def ep_layout_dispatch_noalloc(x, T, H, topk_idx, K, E, R, counts, offsets, tokens_per_rank,
                               is_token_in_rank, num_invalid, layout, cap_or_max_rows, quant,
                               recv_x, recv_scales, slot, recv_src, num_dropped, stream,
                               check=True):
    st = lib().ep_layout_dispatch_noalloc(x, T, H, topk_idx, K, E, R, counts, offsets,
                                          tokens_per_rank, is_token_in_rank, num_invalid, layout,
                                          cap_or_max_rows, quant, recv_x, recv_scales, slot,
                                          recv_src, num_dropped, stream)
    return _check("ep_layout_dispatch_noalloc", st) if check else st


def ep_combine(y, y_rows, H, slot, topk_weights, T, K, out, stream, check=True):
    st = lib().ep_combine(y, y_rows, H, slot, topk_weights, T, K, out, stream)
    return _check("ep_combine", st) if check else st


def ep_dispatch_expert_choice(x, T, H, token_indices, E, C, recv_x, tok_off, tok_ent,
                              num_invalid, ws, ws_bytes, stream, check=True):
    st = lib().ep_dispatch_expert_choice(x, T, H, token_indices, E, C, recv_x, tok_off, tok_ent,
                                         num_invalid, ws, ws_bytes, stream)
    return _check("ep_dispatch_expert_choice", st) if check else st


def ep_combine_expert_choice(y, weights, E, C, H, tok_off, tok_ent, T, out, stream, check=True):
    st = lib().ep_combine_expert_choice(y, weights, E, C, H, tok_off, tok_ent, T, out, stream)
    return _check("ep_combine_expert_choice", st) if check else st


def ep_pack_workspace_bytes(T: int, K: int, E: int, R: int) -> int:
    return lib().ep_pack_workspace_bytes(T, K, E, R)


def ep_pack_by_rank(x, T, H, topk_idx, topk_weights, K, E, R, max_rows, tokens_per_rank,
                    rank_offsets, send_x, send_src, send_idx, send_w, pack_pos, num_dropped, ws,
                    ws_bytes, stream, check=True):
    st = lib().ep_pack_by_rank(x, T, H, topk_idx, topk_weights, K, E, R, max_rows,
                               tokens_per_rank, rank_offsets, send_x, send_src, send_idx, send_w,
                               pack_pos, num_dropped, ws, ws_bytes, stream)
    return _check("ep_pack_by_rank", st) if check else st


def ep_combine_partial(y, y_rows, H, slot, weights, S, K, partial, stream, check=True):
    st = lib().ep_combine_partial(y, y_rows, H, slot, weights, S, K, partial, stream)
    return _check("ep_combine_partial", st) if check else st


def ep_combine_ranks(partial, rows, H, pack_pos, T, R, out, stream, check=True):
    st = lib().ep_combine_ranks(partial, rows, H, pack_pos, T, R, out, stream)
    return _check("ep_combine_ranks", st) if check else st
