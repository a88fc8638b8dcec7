"""CPU oracle for the MoE token dispatch/combine path (ctypes over oracle.c).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package.  It never touches the GPU and the
HIP library never imports it.  The numpy wrappers below only marshal
arguments; all arithmetic is in oracle.c.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# the same source built with -fopenmp: the all-host-cores CPU baseline
_LIB_OMP = os.path.join(_HERE, "liboracle_omp.so")
_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

_lib = None
_lib_omp = None
_override = None


def build(force: bool = True, openmp: bool = False) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (or, with openmp,
    the parallel build oracle/liboracle_omp.so)."""
    out = _LIB_OMP if openmp else _LIB
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        extra = ["-fopenmp"] if openmp else []
        subprocess.run(["gcc", *_CFLAGS, *extra, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


def lib():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        # ORACLE_LIB names another build of oracle.c: the mutation test loads
        # deliberately broken copies this way to show that the pins catch them
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
        _lib = _load(path)
    return _lib


@contextlib.contextmanager
def all_cores():
    """Within the block, every oracle call runs on the -fopenmp build of the
    same source (its token-major loops in parallel over all host cores).
    Yields the number of threads it uses."""
    global _lib_omp, _override
    if _lib_omp is None:
        if not os.path.exists(_LIB_OMP) or os.path.getmtime(_LIB_OMP) < os.path.getmtime(_SRC):
            build(openmp=True)
        _lib_omp = _load(_LIB_OMP)
    prev, _override = _override, _lib_omp
    try:
        yield int(_lib_omp.oracle_max_threads())
    finally:
        _override = prev


def _load(path):
    L = ctypes.CDLL(path)
    L.oracle_max_threads.argtypes = []
    L.oracle_max_threads.restype = ctypes.c_int
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_bf16_to_f32.restype = ctypes.c_float
    L.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
    L.oracle_bf16_from_f64.restype = ctypes.c_uint16
    L.oracle_e4m3_from_f32.argtypes = [ctypes.c_float]
    L.oracle_e4m3_from_f32.restype = ctypes.c_uint8
    L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_to_f32.restype = ctypes.c_float
    L.oracle_e4m3_from_f32_array.argtypes = [_P, _P, _I64]
    L.oracle_e5m2_from_f32_array.argtypes = [_P, _P, _I64]
    L.oracle_e2m1_from_f32_array.argtypes = [_P, _P, _I64]
    L.oracle_e5m2_to_f32.argtypes = [ctypes.c_uint8]
    L.oracle_e5m2_to_f32.restype = ctypes.c_float
    L.oracle_e2m1_to_f32.argtypes = [ctypes.c_uint8]
    L.oracle_e2m1_to_f32.restype = ctypes.c_float
    L.oracle_int8_from_f32.argtypes = [ctypes.c_float]
    L.oracle_int8_from_f32.restype = ctypes.c_int8
    L.oracle_dispatch_token_quant.argtypes = [_P, _I, _I, _P, _I, _I, _P, _P]
    L.oracle_dispatch_mx.argtypes = [_P, _I, _I, _P, _I, _I, _P, _P]
    L.oracle_bf16_from_f64_array.argtypes = [_P, _P, _I64]
    L.oracle_layout.argtypes = [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P]
    L.oracle_slots.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P]
    L.oracle_dispatch_bf16.argtypes = [_P, _I, _I, _P, _I, _P]
    L.oracle_dispatch_fp8.argtypes = [_P, _I, _I, _P, _I, _P, _P]
    L.oracle_combine.argtypes = [_P, _I, _P, _P, _I, _I, _P]
    L.oracle_ec_dispatch.argtypes = [_P, _I, _I, _P, _I, _I, _P, _P]
    L.oracle_ec_invert.argtypes = [_P, _I, _I, _I, _P, _P]
    L.oracle_ec_combine.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _I, _P]
    L.oracle_rank_pack.argtypes = [_P, _I, _I, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                   _P]
    L.oracle_combine_partial.argtypes = [_P, _I, _P, _P, _I, _I, _P]
    L.oracle_combine_ranks.argtypes = [_P, _I, _I, _P, _I, _I, _P]
    for f in ("oracle_layout", "oracle_slots", "oracle_dispatch_bf16", "oracle_dispatch_fp8",
              "oracle_combine", "oracle_ec_dispatch", "oracle_ec_invert", "oracle_ec_combine",
              "oracle_e4m3_from_f32_array", "oracle_bf16_from_f64_array",
              "oracle_e5m2_from_f32_array", "oracle_e2m1_from_f32_array",
              "oracle_dispatch_token_quant", "oracle_dispatch_mx", "oracle_rank_pack",
              "oracle_combine_partial", "oracle_combine_ranks"):
        getattr(L, f).restype = None
    return L


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data if a is not None else None


# ---------------------------------------------------------------- formats
def e4m3_from_f32(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e4m3_from_f32_array(_p(v), _p(out), v.size)
    return out


def e4m3_to_f32(code: int) -> float:
    return lib().oracle_e4m3_to_f32(int(code))


def e5m2_from_f32(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e5m2_from_f32_array(_p(v), _p(out), v.size)
    return out


def e5m2_to_f32(code: int) -> float:
    return lib().oracle_e5m2_to_f32(int(code))


def e2m1_from_f32(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_e2m1_from_f32_array(_p(v), _p(out), v.size)
    return out


def e2m1_to_f32(code: int) -> float:
    return lib().oracle_e2m1_to_f32(int(code))


def int8_from_f32(v: float) -> int:
    return int(lib().oracle_int8_from_f32(float(v)))


def bf16_from_f64(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_from_f64_array(_p(v), _p(out), v.size)
    return out


# ---------------------------------------------------------------- token choice
def layout(topk_idx: np.ndarray, E: int, R: int = 1):
    """-> dict(counts [E], offsets [E+1], tokens_per_rank [R],
    is_token_in_rank [T,R] uint8, num_invalid int)."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    tpr = np.empty(R, np.int32)
    itr = np.empty((T, R), np.uint8)
    ninv = np.zeros(1, np.int32)
    lib().oracle_layout(_p(idx), T, K, E, R, _p(counts), _p(offsets), _p(tpr), _p(itr), _p(ninv))
    return dict(counts=counts, offsets=offsets, tokens_per_rank=tpr,
                is_token_in_rank=itr, num_invalid=int(ninv[0]))


def slots(topk_idx: np.ndarray, E: int, padded: bool, cap_or_max_rows: int):
    """-> (slot [T,K] int32, recv_src [rows] int32 (-2 where unwritten), num_dropped)."""
    idx = _c(topk_idx, np.int32)
    T, K = idx.shape
    rows = E * cap_or_max_rows if padded else cap_or_max_rows
    slot = np.empty((T, K), np.int32)
    src = np.full(rows, -2, np.int32)
    nd = np.zeros(1, np.int32)
    lib().oracle_slots(_p(idx), T, K, E, int(bool(padded)), int(cap_or_max_rows),
                       _p(slot), _p(src), _p(nd))
    return slot, src, int(nd[0])


def dispatch_bf16(x: np.ndarray, slot: np.ndarray, rows: int, recv: np.ndarray = None):
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    K = slot.shape[1] if slot.ndim == 2 else 0
    if recv is None:
        recv = np.zeros((rows, H), np.uint16)
    lib().oracle_dispatch_bf16(_p(x), T, H, _p(slot), K, _p(recv))
    return recv


def dispatch_fp8(x: np.ndarray, slot: np.ndarray, rows: int):
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    K = slot.shape[1]
    q = np.zeros((rows, H), np.uint8)
    s = np.zeros((rows, H // 128), np.float32)
    lib().oracle_dispatch_fp8(_p(x), T, H, _p(slot), K, _p(q), _p(s))
    return q, s


TOKEN_FMT = {"fp8_e4m3_token": 0, "int8_token": 1}
MX_FMT = {"mxfp8_e4m3": 0, "mxfp8_e5m2": 1, "mxfp4_e2m1": 2}


def dispatch_token_quant(x: np.ndarray, slot: np.ndarray, rows: int, mode: str):
    """Per-token scaled quantisation ("fp8_e4m3_token" or "int8_token"):
    -> (codes [rows, H] uint8, scales [rows] float32)."""
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    K = slot.shape[1]
    q = np.zeros((rows, H), np.uint8)
    s = np.zeros(rows, np.float32)
    lib().oracle_dispatch_token_quant(_p(x), T, H, _p(slot), K, TOKEN_FMT[mode], _p(q), _p(s))
    return q, s


def dispatch_mx(x: np.ndarray, slot: np.ndarray, rows: int, mode: str):
    """MX quantisation ("mxfp8_e4m3", "mxfp8_e5m2", "mxfp4_e2m1"):
    -> (codes [rows, H or H/2] uint8, e8m0 scale codes [rows, H/32] uint8)."""
    x = _c(x, np.uint16)
    slot = _c(slot, np.int32)
    T, H = x.shape
    K = slot.shape[1]
    fmt = MX_FMT[mode]
    q = np.zeros((rows, H // 2 if fmt == 2 else H), np.uint8)
    e = np.zeros((rows, H // 32), np.uint8)
    lib().oracle_dispatch_mx(_p(x), T, H, _p(slot), K, fmt, _p(q), _p(e))
    return q, e


def combine(y: np.ndarray, slot: np.ndarray, w=None):
    """y [rows, H] bf16 bits; slot [T, K]; w [T, K] float32 or None."""
    y = _c(y, np.uint16)
    slot = _c(slot, np.int32)
    T, K = slot.shape
    H = y.shape[1]
    wa = _c(w, np.float32) if w is not None else None
    out = np.empty((T, H), np.uint16)
    lib().oracle_combine(_p(y), H, _p(slot), _p(wa), T, K, _p(out))
    return out


# ---------------------------------------------------------------- expert choice
def ec_dispatch(x: np.ndarray, token_indices: np.ndarray, recv: np.ndarray = None):
    x = _c(x, np.uint16)
    ti = _c(token_indices, np.int32)
    T, H = x.shape
    E, C = ti.shape
    if recv is None:
        recv = np.zeros((E, C, H), np.uint16)
    ninv = np.zeros(1, np.int32)
    lib().oracle_ec_dispatch(_p(x), T, H, _p(ti), E, C, _p(recv), _p(ninv))
    return recv, int(ninv[0])


def ec_invert(token_indices: np.ndarray, T: int):
    ti = _c(token_indices, np.int32)
    E, C = ti.shape
    off = np.empty(T + 1, np.int32)
    ent = np.full(E * C, -2, np.int32)
    lib().oracle_ec_invert(_p(ti), E, C, T, _p(off), _p(ent))
    return off, ent


def ec_combine(y: np.ndarray, w: np.ndarray, token_indices: np.ndarray, T: int, tokens=None):
    """y [E, C, H] (or [E*C, H]) bf16 bits; w [E, C] float32."""
    ti = _c(token_indices, np.int32)
    E, C = ti.shape
    y = _c(y, np.uint16).reshape(E * C, -1)
    H = y.shape[1]
    w = _c(w, np.float32)
    tk = _c(tokens, np.int32) if tokens is not None else None
    n = len(tk) if tk is not None else T
    out = np.empty((n, H), np.uint16)
    lib().oracle_ec_combine(_p(y), _p(w), _p(ti), E, C, H, T, _p(tk), n, _p(out))
    return out


# ---------------------------------------------------------------- one rank's share
def rank_pack(x: np.ndarray, topk_idx: np.ndarray, w, E: int, R: int, max_rows: int = None):
    """Sender pack keyed by (destination rank, token) -> dict(rank_offsets
    [R+1], send_x [rows, H], send_src [rows], send_idx [rows, K], send_w
    [rows, K] (unit weights where w is None), pack_pos [T, R], num_dropped).
    Rows past the last kept one keep zeros in send_x, -2 in send_src, -3 in
    send_idx and nan in send_w."""
    x = _c(x, np.uint16)
    idx = _c(topk_idx, np.int32)
    T, H = x.shape
    K = idx.shape[1]
    if max_rows is None:
        max_rows = T * min(K, R)
    wa = _c(w, np.float32) if w is not None else None
    off = np.empty(R + 1, np.int32)
    sx = np.zeros((max_rows, H), np.uint16)
    src = np.full(max_rows, -2, np.int32)
    sidx = np.full((max_rows, K), -3, np.int32)
    sw = np.full((max_rows, K), np.nan, np.float32)
    pos = np.empty((T, R), np.int32)
    nd = np.zeros(1, np.int32)
    lib().oracle_rank_pack(_p(x), T, H, _p(idx), _p(wa), K, E, R, max_rows, _p(off), _p(sx),
                           _p(src), _p(sidx), _p(sw), _p(pos), _p(nd))
    return dict(rank_offsets=off, send_x=sx, send_src=src, send_idx=sidx, send_w=sw,
                pack_pos=pos, num_dropped=int(nd[0]))


def combine_partial(y: np.ndarray, slot: np.ndarray, w=None):
    """y [rows, H] bf16 bits; slot [S, K]; w [S, K] float32 or None ->
    partial [S, H] float32."""
    y = _c(y, np.uint16)
    slot = _c(slot, np.int32)
    S, K = slot.shape
    H = y.shape[1]
    wa = _c(w, np.float32) if w is not None else None
    out = np.empty((S, H), np.float32)
    lib().oracle_combine_partial(_p(y), H, _p(slot), _p(wa), S, K, _p(out))
    return out


def combine_ranks(partial: np.ndarray, pack_pos: np.ndarray):
    """partial [rows, H] float32; pack_pos [T, R] -> out [T, H] bf16 bits."""
    pa = _c(partial, np.float32)
    pos = _c(pack_pos, np.int32)
    T, R = pos.shape
    rows, H = pa.shape
    out = np.empty((T, H), np.uint16)
    lib().oracle_combine_ranks(_p(pa), rows, H, _p(pos), T, R, _p(out))
    return out
