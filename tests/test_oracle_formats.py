"""Pins for the oracle's number formats: the E4M3 encoder and the bf16 rounding.

Each check compares the oracle with something other than itself: hand-derived
codes, a brute-force nearest-code search, and torch's own casts.
"""
import os

import numpy as np
import pytest
import torch

import brute
import golden_io
import oracle


def test_e4m3_golden_codes():
    for v, code in golden_io.read_table("e4m3_codes.txt"):
        got = int(oracle.e4m3_from_f32(np.array([v], np.float32))[0])
        assert got == code, (v, hex(got), hex(code))


def test_e4m3_decode_table_matches_definition():
    tab = brute.e4m3_table()
    for c in range(256):
        got = oracle.e4m3_to_f32(c)
        if np.isnan(tab[c]):
            assert np.isnan(got)
        else:
            assert got == tab[c], c
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6


def _boundary_values():
    """Every code value, every midpoint between neighbouring codes and a few
    values past 448, plus the fp32 values 1..3 ulps either side of each, both
    signs."""
    tab = brute.e4m3_table()
    pos = np.sort(tab[:127][~np.isnan(tab[:127])])
    mids = (pos[:-1] + pos[1:]) / 2
    base = np.concatenate([pos, mids, [456.0, 463.99, 464.0, 470.0, 500.0]]).astype(np.float32)
    ext = [base]
    up, dn = base.copy(), base.copy()
    for _ in range(3):
        up = np.nextafter(up, np.float32(np.inf))
        dn = np.nextafter(dn, np.float32(-np.inf))
        ext += [up, dn]
    v = np.concatenate(ext).astype(np.float32)
    return np.concatenate([v, -v])


def test_e4m3_vs_nearest_code_search_boundaries():
    v = _boundary_values()
    got = oracle.e4m3_from_f32(v)
    ref = brute.e4m3_nearest(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(ref[i])) for i in bad[:10]]


def test_e4m3_vs_nearest_code_search_random():
    rng = np.random.default_rng(11)
    # log-uniform magnitudes over the whole e4m3 range and a bit beyond, random signs
    mag = np.exp2(rng.uniform(-13, 9.0, 400_000)).astype(np.float32)
    v = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    for lo in range(0, v.size, 50_000):
        chunk = v[lo:lo + 50_000]
        got = oracle.e4m3_from_f32(chunk)
        ref = brute.e4m3_nearest(chunk)
        assert np.array_equal(got, ref)


def _torch_e4m3(v):
    return torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("stride", [1 if os.environ.get("EP_EXHAUSTIVE") else 7])
def test_e4m3_vs_torch_cast_exhaustive(stride):
    """Every non-negative fp32 pattern below 464 (the satfinite boundary; torch
    returns NaN above it) against torch's float8_e4m3fn cast, which rounds to
    nearest even.  stride 1 (EP_EXHAUSTIVE=1) covers all 1.14e9 patterns;
    the default walks every 7th pattern, which still visits every binade and
    every rounding boundary's neighbourhood many times."""
    top = int(np.array([464.0], np.float32).view(np.uint32)[0])
    step = 1 << 24
    for lo in range(0, top, step * stride):
        bits = np.arange(lo, min(lo + step * stride, top), stride, dtype=np.uint32)
        v = bits.view(np.float32)
        got = oracle.e4m3_from_f32(v)
        ref = _torch_e4m3(v)
        if not np.array_equal(got, ref):
            i = int(np.nonzero(got != ref)[0][0])
            raise AssertionError((float(v[i]), hex(got[i]), hex(ref[i])))
        # sign symmetry on the same patterns
        gotn = oracle.e4m3_from_f32(-v)
        assert np.array_equal(gotn, got | 0x80)


def test_bf16_golden():
    for v, code in golden_io.read_table("bf16_round.txt"):
        got = int(oracle.bf16_from_f64(np.array([v]))[0])
        assert got == code, (v.hex(), hex(got), hex(code))


def test_bf16_vs_torch_cast_on_fp32_inputs():
    """For values that are fp32 numbers, rounding to bf16 must equal torch's
    float32 -> bfloat16 cast (round to nearest even)."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    # add exact ties: low 16 bits 0x8000
    ties = (bits & 0xFFFF0000) | 0x8000
    allb = np.concatenate([bits, ties])
    v = allb.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.3e38)]
    got = oracle.bf16_from_f64(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_vs_neighbour_search_on_f64_inputs():
    """Doubles between bf16 neighbours, including exact ties and values a hair
    off a tie (which an fp32 intermediate would collapse onto the tie)."""
    rng = np.random.default_rng(6)
    base = rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))
    b16 = brute.bf16_nearest_f64(base)
    lo = brute.bf16_to_f64(b16)
    step = np.exp2(np.floor(np.log2(np.abs(lo))) - 7)      # one bf16 ulp at lo
    ties = lo + np.sign(base) * step / 2
    off = ties + np.sign(base) * step * 2.0 ** -30
    off2 = ties - np.sign(base) * step * 2.0 ** -30
    v = np.concatenate([base, ties, off, off2, [2.0 ** -140, -(2.0 ** -133) * 1.5]])
    got = oracle.bf16_from_f64(v)
    ref = brute.bf16_nearest_f64(v)
    assert np.array_equal(got, ref)
