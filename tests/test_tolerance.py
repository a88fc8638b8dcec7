"""The combine tolerance check itself (CPU): every non-finite result fails,
and the bound sits exactly where |gpu - oracle| <= 2^-7 |oracle| + 1e-3
puts it."""
import numpy as np
import pytest

import tolerance as T


def _bits(v):
    """bf16 bits of float32 values that are exactly representable in bf16."""
    a = np.asarray(v, np.float32).view(np.uint32)
    assert ((a & 0xFFFF) == 0).all()
    return (a >> 16).astype(np.uint16)


REF = _bits([1.0, -2.5, 0.0, 384.0, -0.0078125, 0.5])


@pytest.mark.parametrize("planted", [0x7FC0, 0xFFC0, 0x7F81, 0x7F80, 0xFF80])
@pytest.mark.parametrize("where", [0, 2, 5])
def test_non_finite_result_fails(planted, where):
    """quiet NaN, negative NaN, signalling NaN, +Inf, -Inf against finite
    oracle values, including an oracle zero (where the bound is 1e-3)."""
    got = REF.copy()
    got[where] = planted
    with pytest.raises(AssertionError):
        T.assert_combine_close(got, REF)
    assert T.combine_bad(got, REF)[0].tolist() == [where]


@pytest.mark.parametrize("planted", [0x7FC0, 0x7F80, 0xFF80])
def test_non_finite_oracle_fails(planted):
    """An oracle value that is not finite (out of contract) never passes,
    even against the same bits, and not against any finite value either
    (where |oracle| = inf would make the bound itself infinite)."""
    ref = REF.copy()
    ref[1] = planted
    with pytest.raises(AssertionError):
        T.assert_combine_close(ref.copy(), ref)
    for finite in (0x0000, 0x3F80, 0x7F7F, 0xFF7F):      # 0, 1, +-largest finite
        got = ref.copy()
        got[1] = finite
        assert T.combine_bad(got, ref)[0].tolist() == [1], hex(finite)


def test_equal_passes_and_2d():
    T.assert_combine_close(REF.copy(), REF)
    g = np.tile(REF, (3, 1))
    T.assert_combine_close(g, g.copy())
    g2 = g.copy()
    g2[2, 3] = 0x7FC0
    assert [ix for ix in zip(*T.combine_bad(g2, g))] == [(2, 3)]


def test_bound_edges():
    """At |oracle| = 384 the bound is 3 + 1e-3: 386 (2 off) passes, 388 (4
    off) fails.  At oracle 0 the bound is 1e-3: 2^-10 passes, 2^-9 fails."""
    ref = _bits([384.0, 0.0, 0.0])
    T.assert_combine_close(_bits([386.0, 2.0 ** -10, -(2.0 ** -10)]), ref)
    for bad in ([388.0, 0.0, 0.0], [384.0, 2.0 ** -9, 0.0], [384.0, 0.0, -(2.0 ** -9)]):
        with pytest.raises(AssertionError):
            T.assert_combine_close(_bits(bad), ref)


def test_shape_mismatch_fails():
    with pytest.raises(AssertionError):
        T.assert_combine_close(REF[:3], REF)


@pytest.mark.parametrize("planted", [np.nan, -np.nan, np.inf, -np.inf])
def test_f32_non_finite_fails(planted):
    ref = np.array([1.0, -2.5, 0.0, 384.0], np.float32)
    T.assert_f32_close(ref.copy(), ref)
    for where in range(4):
        got = ref.copy()
        got[where] = planted
        with pytest.raises(AssertionError):
            T.assert_f32_close(got, ref)
        # the non-finite value on the oracle side, against finite results
        with pytest.raises(AssertionError):
            T.assert_f32_close(ref.copy(), got)


def test_f32_bound_edges():
    ref = np.array([384.0, 0.0], np.float32)
    T.assert_f32_close(np.array([386.9, 0.00099], np.float32), ref)
    with pytest.raises(AssertionError):
        T.assert_f32_close(np.array([387.1, 0.0], np.float32), ref)
    with pytest.raises(AssertionError):
        T.assert_f32_close(np.array([384.0, 0.0011], np.float32), ref)
