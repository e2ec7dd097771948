"""Pins of the oracle's chunked-prefill functions (no GPU): the range merged
chunk by chunk and the codes on a given range.

Pages: QbitAI article on CalibQuant, section "Method" part 1 (the uniform
quantizer's range is refined per channel over the tokens of one head, values
are rounded to the nearest level); the 1-bit codebook holds the channel's
minimum and maximum (part 3).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rand(shape, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * rng.uniform(0.5, 2, shape[-1]) + rng.standard_normal(shape[-1])
    return x.astype(dtype)


def _ranges(x, seed):
    """The data's own range, a narrower one (values fall outside), a wider
    one, and one with degenerate and inverted channels."""
    rng = np.random.default_rng(seed)
    lo = x.min(axis=0).astype(np.float32)
    hi = x.max(axis=0).astype(np.float32)
    w = hi - lo
    narrow = (lo + np.float32(0.3) * w, hi - np.float32(0.25) * w)
    wide = (lo - np.float32(0.5) * w, hi + np.float32(0.125) * w)
    odd_lo, odd_hi = lo.copy(), hi.copy()
    odd_hi[0] = odd_lo[0]                                  # mx == mn
    odd_lo[1], odd_hi[1] = hi[1], lo[1]                    # mx < mn
    odd_lo[2] = odd_hi[2] = np.float32(rng.standard_normal())
    return [(lo, hi), narrow, wide, (odd_lo, odd_hi)]


# ---- given-range codes: nearest level by exhaustive search ----------------

@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_given_range_is_nearest_level(bits, dtype):
    """Every code is the nearest of the 2^b levels of the given range (ties
    to the even level), found by exhaustive search in exact arithmetic; values
    outside the range land on an end level."""
    x = _rand((9, 6), dtype, 100 + bits)
    for mn, mx in _ranges(x, bits):
        codes, scale, minv = oracle.quantize_with_range(x, mn, mx, bits)
        brute = oracle.quantize_brute_range(x.astype(np.float64).tolist(), mn.astype(np.float64).tolist(),
                                            mx.astype(np.float64).tolist(), bits)
        assert codes.tolist() == brute
        assert codes.min() >= 0 and codes.max() <= (1 << bits) - 1
        assert np.array_equal(minv, mn)
        L = (1 << bits) - 1
        for j in range(x.shape[1]):
            if mx[j] > mn[j]:
                exact = (Fraction(float(mx[j])) - Fraction(float(mn[j]))) / L
                assert abs(Fraction(float(scale[j])) - exact) <= abs(Fraction(float(np.spacing(scale[j])))) / 2
            else:
                assert scale[j] == 0 and not codes[:, j].any()


def test_given_range_ties_exact():
    """Values exactly on a half-level go to the even code; on a 2-bit grid
    over [0, 3] the levels are 0, 1, 2, 3."""
    x = np.array([[-1.0], [0.5], [1.5], [2.5], [3.0], [7.0], [1.25], [2.75]], np.float16)
    codes, scale, minv = oracle.quantize_with_range(x, np.array([0.0], np.float32), np.array([3.0], np.float32), 2)
    assert codes[:, 0].tolist() == [0, 0, 2, 2, 3, 3, 1, 3]
    assert scale.tolist() == [1.0] and minv.tolist() == [0.0]


def test_one_bit_is_midpoint_test():
    """b = 1: the code is 1 exactly when x lies strictly above the midpoint
    of the given range (the midpoint itself rounds half to even, to 0)."""
    x = _rand((64, 16), np.float16, 7)
    for mn, mx in _ranges(x, 7):
        codes, _, _ = oracle.quantize_with_range(x, mn, mx, 1)
        for j in range(16):
            mid = (Fraction(float(mn[j])) + Fraction(float(mx[j]))) / 2
            want = [int(mx[j] > mn[j] and Fraction(float(v)) > mid) for v in x[:, j]]
            assert codes[:, j].tolist() == want
    # a value exactly on the midpoint
    codes, _, _ = oracle.quantize_with_range(np.array([[1.0], [1.0009765625]], np.float16),
                                             np.array([0.0], np.float32), np.array([2.0], np.float32), 1)
    assert codes[:, 0].tolist() == [0, 1]


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_own_range_equals_one_shot(bits, dtype):
    """With the data's own range, the given-range quantizer is the one-shot
    quantizer: same codes, scale and minimum."""
    x = _rand((200, 32), dtype, 200 + bits)
    c1, s1, m1, _ = oracle.quantize_unit(x, bits)
    c2, s2, m2 = oracle.quantize_with_range(x, x.min(axis=0), x.max(axis=0), bits)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2) and np.array_equal(m1, m2)


def test_non_f16_range_over_f16_data():
    """A float32 range that is not on the float16 grid is still decided
    exactly (the midpoint of -2^-30 and 1 lies just below 1/2)."""
    x = np.array([[0.5], [0.49951171875], [0.50048828125]], np.float16)
    codes, scale, _ = oracle.quantize_with_range(x, np.array([-2.0 ** -30], np.float32), np.array([1.0], np.float32), 1)
    assert codes[:, 0].tolist() == [1, 0, 1]
    assert scale[0] == np.float32(1.0 + 2.0 ** -30)


# ---- the range merged chunk by chunk ---------------------------------------

@pytest.mark.parametrize("dtype", [np.float16, np.float32])
def test_chunked_range_is_whole_range(dtype):
    """Min and max are associative: after the last chunk the merged range is
    the range of the whole segment, whatever the chunking."""
    x = _rand((1000, 24), dtype, 11)
    for cuts in ([0, 1000], [0, 1, 2, 999, 1000], [0, 128, 512, 600, 1000], list(range(0, 1001, 100))):
        mn = mx = None
        for a, b in zip(cuts[:-1], cuts[1:]):
            mn, mx, _ = oracle.range_update(mn, mx, x[a:b], reset=mn is None)
        assert np.array_equal(mn, x.min(axis=0).astype(np.float32))
        assert np.array_equal(mx, x.max(axis=0).astype(np.float32))


def test_grew_flag():
    """grew is True exactly when a channel's stored range changes."""
    x = np.array([[0.0, 1.0], [2.0, -1.0]], np.float16)
    mn, mx, g = oracle.range_update(None, None, x, reset=True)
    assert g and mn.tolist() == [0.0, -1.0] and mx.tolist() == [2.0, 1.0]
    mn2, mx2, g = oracle.range_update(mn, mx, np.array([[1.0, 0.5], [0.0, -1.0]], np.float16), reset=False)
    assert not g and np.array_equal(mn2, mn) and np.array_equal(mx2, mx)
    _, _, g = oracle.range_update(mn, mx, np.array([[1.0, 1.5]], np.float16), reset=False)
    assert g
    _, _, g = oracle.range_update(mn, mx, np.array([[-0.5, 0.0]], np.float16), reset=False)
    assert g
    _, _, g = oracle.range_update(np.array([0.0, 0.0], np.float32), np.array([1.0, 1.0], np.float32),
                                  np.array([[-0.0, 1.0]], np.float16), reset=False)
    assert not g                                              # -0 == +0 widens nothing


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_chunked_prefill_equals_one_shot(bits):
    """Gather the range chunk by chunk, then code every chunk on the final
    range: the cache equals the one-shot quantization of the segment."""
    x = _rand((768, 16), np.float16, 300 + bits)
    mn = mx = None
    for a in range(0, 768, 256):
        mn, mx, _ = oracle.range_update(mn, mx, x[a:a + 256], reset=a == 0)
    parts = [oracle.quantize_with_range(x[a:a + 256], mn, mx, bits) for a in range(0, 768, 256)]
    c1, s1, m1, _ = oracle.quantize_unit(x, bits)
    assert np.array_equal(np.concatenate([p[0] for p in parts]), c1)
    for p in parts:
        assert np.array_equal(p[1], s1) and np.array_equal(p[2], m1)


def test_stale_range_codes_differ_then_repack_fixes():
    """Codes written on a range that a later chunk widens are stale; coding
    them again on the widened range gives the one-shot result."""
    x = _rand((512, 8), np.float16, 5)
    x[300, 3] = np.float16(50.0)                            # the second chunk widens channel 3
    mn, mx, _ = oracle.range_update(None, None, x[:256], reset=True)
    stale, _, _ = oracle.quantize_with_range(x[:256], mn, mx, 1)
    mn, mx, grew = oracle.range_update(mn, mx, x[256:], reset=False)
    assert grew
    fresh, _, _ = oracle.quantize_with_range(x[:256], mn, mx, 1)
    one, _, _, _ = oracle.quantize_unit(x, 1)
    assert np.array_equal(fresh, one[:256])
    assert not np.array_equal(stale[:, 3], fresh[:, 3])
