"""The combine tolerance, per element on fp32-widened bf16 values:

    |gpu - oracle| <= 2^-7 * |oracle| + 1e-3

An element passes only when both values are finite and that comparison is
true.  A NaN on either side fails (NaN <= anything is false), and so does an
infinity on either side: an infinite oracle value is out of contract, and
against it the bound itself would be infinite.  numpy only: the check itself
is tested on the CPU.
"""
import numpy as np

REL = 2.0 ** -7
ABS = 1e-3


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def combine_bad(got_bits, ref_bits):
    """Indices (np.nonzero form) of elements outside the tolerance."""
    g = bf16_f64(got_bits)
    r = bf16_f64(ref_bits)
    if g.shape != r.shape:
        raise AssertionError(f"shape {g.shape} against {r.shape}")
    with np.errstate(invalid="ignore", over="ignore"):
        ok = np.isfinite(g) & np.isfinite(r) & (np.abs(g - r) <= REL * np.abs(r) + ABS)
    return np.nonzero(~ok)


def assert_combine_close(got_bits, ref_bits, what=""):
    bad = combine_bad(got_bits, ref_bits)
    if bad[0].size:
        g, r = bf16_f64(got_bits), bf16_f64(ref_bits)
        raise AssertionError((what, int(bad[0].size),
                              [(tuple(int(i) for i in ix), g[ix], r[ix])
                               for ix in list(zip(*bad))[:5]]))


def f32_bad(got, ref):
    """The same bound on fp32 values (the partial sums of the exchange)."""
    g = np.asarray(got, np.float32).astype(np.float64)
    r = np.asarray(ref, np.float32).astype(np.float64)
    if g.shape != r.shape:
        raise AssertionError(f"shape {g.shape} against {r.shape}")
    with np.errstate(invalid="ignore", over="ignore"):
        ok = np.isfinite(g) & np.isfinite(r) & (np.abs(g - r) <= REL * np.abs(r) + ABS)
    return np.nonzero(~ok)


def assert_f32_close(got, ref, what=""):
    bad = f32_bad(got, ref)
    if bad[0].size:
        g, r = np.asarray(got), np.asarray(ref)
        raise AssertionError((what, int(bad[0].size),
                              [(tuple(int(i) for i in ix), g[ix], r[ix])
                               for ix in list(zip(*bad))[:5]]))
