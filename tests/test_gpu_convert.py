"""Exhaustive GPU check of the dispatch kernel's element arithmetic.

The dispatch kernel encodes with gfx950's conversion instructions and
divides by a shared scale with one reciprocal and one correction step
(`ep_common.h`).  `tests/hwcheck/convert_check.hip` compares exactly those
helpers, on the GPU, with software definitions over whole input domains:
every finite fp32 input for the E4M3 / E5M2 / E2M1 codes (each byte or nibble
position), every MX block value for the scaled E2M1 conversion, and every
(bf16 amax, bf16 |x| <= amax) pair for the division at s = amax/448 and
amax/127.  The formats are those of "DeepEP-Ascend" README, Quantization
Modes in Normal Dispatch (float8_e4m3fn, float8_e5m2, MXFP4 e2m1, INT8).

Here every check must report zero mismatches, and each must have seen the
number of cases its domain holds (counted independently below).
"""
import ctypes
import os
import time

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hwcheck", "libconvert_check.so")

CHECKS = ["e4m3 |v|<464", "e4m3 med3", "e5m2 |v|<61440", "e5m2 med3", "e2m1 fp32",
          "e2m1 mx scaled", "x/448 e4m3 code", "x/127 int8 code", "x/448 fp32 |q|>=2^-11",
          "x/127 fp32 |q|>=2^-11", "x/448 hw e4m3 code"]


def _finite_fp32_below(bits):
    """Number of fp32 patterns (both signs) with magnitude pattern < bits."""
    return 2 * bits


def _mx_e2m1_cases():
    b = np.arange(65536, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]                       # finite bf16
    ax = np.abs((b << 16).view(np.float32).astype(np.float64))
    return int(sum(np.count_nonzero(ax * 2.0 ** -e < 8.0) for e in range(-127, 126)))


def _div_pairs():
    ab = np.arange(1, 0x7F80, dtype=np.int64)
    return int((2 * (ab + 1)).sum())                    # |x| pattern 0..ab, both signs


def test_conversions_and_division_exhaustive():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is missing: run __graft_entry__.build() first")
    import torch
    assert torch.cuda.is_available()
    torch.cuda.init()
    lib = ctypes.CDLL(LIB)
    lib.convert_check.argtypes = [ctypes.c_void_p]
    lib.convert_check.restype = ctypes.c_int
    n = lib.convert_check_num_counters()
    assert n == 2 * len(CHECKS)
    counts = (ctypes.c_ulonglong * n)()
    print("[case] exhaustive conversion and division check", flush=True)
    t0 = time.time()
    rc = lib.convert_check(ctypes.cast(counts, ctypes.c_void_p))
    print(f"  {time.time() - t0:.1f} s", flush=True)
    assert rc == 0, f"HIP error {rc}"
    bad = {c: counts[i] for i, c in enumerate(CHECKS)}
    seen = {c: counts[len(CHECKS) + i] for i, c in enumerate(CHECKS)}
    print(bad, seen, flush=True)
    assert all(v == 0 for v in bad.values()), bad

    finite = _finite_fp32_below(0x7F800000)
    pairs = _div_pairs()
    assert seen["e4m3 |v|<464"] == _finite_fp32_below(0x43E80000)
    assert seen["e4m3 med3"] == finite
    assert seen["e5m2 |v|<61440"] == _finite_fp32_below(0x47700000)
    assert seen["e5m2 med3"] == finite
    assert seen["e2m1 fp32"] == finite
    assert seen["e2m1 mx scaled"] == _mx_e2m1_cases()
    assert seen["x/448 e4m3 code"] == pairs
    assert seen["x/127 int8 code"] == pairs
    assert seen["x/448 hw e4m3 code"] == pairs
    assert 0 < seen["x/448 fp32 |q|>=2^-11"] < pairs
    assert 0 < seen["x/127 fp32 |q|>=2^-11"] < pairs
