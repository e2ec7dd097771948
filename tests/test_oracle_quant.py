"""Pins of the oracle's quantizer and packer against what the pages and the
mathematics fix (no GPU).

Pages: QbitAI article on CalibQuant, section "Method" part 1 (channel-wise
uniform integer quantization), part 2 (only b-bit integers are stored; e.g.
2-bit values are 0, 1, 2, 3), part 3 (the 1-bit codebook holds min and max).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import ROLE_K, ROLE_V, kv_numpy

HERE = os.path.dirname(__file__)


def _rand(shape, dtype, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape) * rng.uniform(0.5, 2, shape[-1]) + rng.standard_normal(shape[-1])
    return x.astype(dtype)


# ---- golden, hand-derived -------------------------------------------------

def test_golden_hand_example():
    g = json.load(open(os.path.join(HERE, "golden", "quantize_hand.json")))
    x = np.array(g["x"], np.float16)
    for case in g["cases"]:
        codes, scale, minv, _ = oracle.quantize_unit(x, case["bits"])
        assert codes.tolist() == case["codes"]
        assert scale.tolist() == case["scale"]
        assert minv.tolist() == case["min"]
    x32 = x.astype(np.float32)
    for case in g["cases"]:
        codes, scale, minv, _ = oracle.quantize_unit(x32, case["bits"])
        assert codes.tolist() == case["codes"]


# ---- P1: codebook ---------------------------------------------------------

@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_codes_in_codebook(bits, dtype):
    x = _rand((64, 16), dtype, bits)
    codes, *_ = oracle.quantize_unit(x, bits)
    L = (1 << bits) - 1
    assert codes.min() == 0 and codes.max() == L
    assert set(np.unique(codes)) <= set(range(L + 1))
    if bits == 2:
        assert set(np.unique(codes)) == {0, 1, 2, 3}


# ---- P2: min and max are reproduced exactly --------------------------------

@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_endpoints_exact(bits, dtype):
    x = _rand((40, 12), dtype, 10 + bits)
    codes, scale, minv, _ = oracle.quantize_unit(x, bits)
    L = (1 << bits) - 1
    for j in range(x.shape[1]):
        lo, hi = int(np.argmin(x[:, j])), int(np.argmax(x[:, j]))
        assert codes[lo, j] == 0 and codes[hi, j] == L
        mn, mx = Fraction(float(x[:, j].min())), Fraction(float(x[:, j].max()))
        step = (mx - mn) / L
        assert mn + 0 * step == Fraction(float(x[lo, j]))
        assert mn + L * step == Fraction(float(x[hi, j]))
        assert float(minv[j]) == float(x[lo, j])


# ---- P3: reconstruction error is at most half a step -----------------------

@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_half_step_bound(bits, dtype):
    x = _rand((50, 9), dtype, 20 + bits)
    codes, _, _, scale_exact = oracle.quantize_unit(x, bits)
    for j in range(x.shape[1]):
        mn = Fraction(float(x[:, j].min()))
        mx = Fraction(float(x[:, j].max()))
        step = (mx - mn) / ((1 << bits) - 1)
        for i in range(x.shape[0]):
            err = abs(Fraction(float(x[i, j])) - (mn + codes[i, j] * step))
            assert err <= step / 2


# ---- P4: brute-force nearest level, including forced ties ------------------

def _tie_block(bits, dtype):
    """Channels whose values sit exactly on half-levels between mn and mx."""
    L = (1 << bits) - 1
    cols = []
    for mn, span in ((0.0, float(L)), (-3.0, 2.0 * L), (1.5, 0.5 * L)):
        step = span / L
        vals = [mn, mn + span] + [mn + (k + 0.5) * step for k in range(min(L, 6))]
        vals += [mn + k * step for k in range(min(L + 1, 4))]
        cols.append(vals[:8])
    return np.array(cols, dtype=np.float64).T.astype(dtype)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_matches_brute_force(bits, dtype):
    for x in (_rand((12, 5), dtype, 30 + bits), _tie_block(bits, dtype)):
        codes, _, _, _ = oracle.quantize_unit(x, bits)
        ref, _, _ = oracle.quantize_brute(x.astype(np.float64).tolist(), bits)
        assert codes.tolist() == ref


def test_ties_go_to_even():
    x = _tie_block(2, "float16")
    codes, *_ = oracle.quantize_unit(x, 2)
    # column 0: mn 0, mx 3, values k + 0.5 for k = 0, 1, 2 -> even neighbours 0, 2, 2
    assert codes[2:5, 0].tolist() == [0, 2, 2]


def test_degenerate_channel():
    x = np.full((7, 3), 1.25, np.float16)
    x[:, 1] = np.arange(7)
    codes, scale, minv, _ = oracle.quantize_unit(x, 1)
    assert (codes[:, 0] == 0).all() and scale[0] == 0 and minv[0] == np.float32(1.25)
    assert codes[:, 1].tolist() == [0, 0, 0, 0, 1, 1, 1]


def test_empty_unit():
    codes, scale, minv, _ = oracle.quantize_unit(np.zeros((0, 4), np.float16), 1)
    assert codes.shape == (0, 4) and (scale == 0).all() and (minv == 0).all()


def test_fp16_wide_exponent_spread():
    """Values spanning subnormals to the fp16 maximum stay exact."""
    x = np.array([[6.0e-8], [65504.0], [-65504.0], [3.0e-5], [0.0]], np.float16)
    codes, *_ = oracle.quantize_unit(x, 8)
    ref, _, _ = oracle.quantize_brute(x.astype(np.float64).tolist(), 8)
    assert codes.tolist() == ref


# ---- float32 rounding of the stored scale ---------------------------------

def test_nearest_f32_is_single_rounding():
    mid = Fraction(1) + Fraction(1, 1 << 24)          # halfway between 1 and 1 + 2**-23
    assert oracle.nearest_f32(mid) == np.float32(1.0)  # tie -> even mantissa
    above = mid + Fraction(1, 1 << 60)                 # float64 cannot see the excess
    assert float(above) == float(mid)
    assert oracle.nearest_f32(above) == np.nextafter(np.float32(1), np.float32(2))
    assert oracle.nearest_f32(Fraction(1, 3)) == np.float32(1 / 3)


def test_exact_ints_roundtrip():
    for dt in ("float16", "float32"):
        x = _rand((9, 4), dt, 5)
        X, k = oracle.exact_ints(x)
        for v, I in zip(x.ravel(), X.ravel()):
            assert Fraction(int(I), 1 << k) == Fraction(float(v))


# ---- packed layouts ---------------------------------------------------------

def test_bit_offsets_are_a_partition():
    for bits in (1, 2, 4, 8):
        E = 32 // bits
        used = 0
        for e in range(E):
            field = ((1 << bits) - 1) << oracle.code_bit_offset(e, bits)
            assert used & field == 0
            used |= field
        assert used == 0xFFFFFFFF


def test_pack_hand_words():
    # b=1, K layout, d=32 -> one word per token; channel j at bit 8*(j%4) + j//4
    c = np.zeros((3, 32), np.int64)
    c[0, 5] = 1          # bit 9
    c[1, 31] = 1         # bit 31
    c[2, 4] = 1          # bit 1
    c[2, 0] = 1          # bit 0
    w = oracle.pack(c, 1, "K")
    assert w.shape == (1, 3)
    assert w[0].tolist() == [0x200, 0x80000000, 0x3]
    # b=4, V layout: tokens 0..7 of one channel -> nibble offsets 0,8,16,24,4,12,20,28
    c = np.arange(8, dtype=np.int64).reshape(8, 1) + 1       # codes 1..8
    w = oracle.pack(c, 4, "V")
    assert w.shape == (1, 1)
    assert int(w[0, 0]) == 0x84736251
    # b=8 is plain little-endian bytes
    c = np.array([[1], [2], [3], [250]], np.int64)
    assert int(oracle.pack(c, 8, "V")[0, 0]) == 0xFA030201


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
def test_pack_unpack_roundtrip_and_padding(bits):
    rng = np.random.default_rng(bits)
    n, d = 45, 64
    c = rng.integers(0, 1 << bits, (n, d))
    for layout in ("K", "V"):
        w = oracle.pack(c, bits, layout)
        assert w.dtype == np.uint32
        assert (oracle.unpack(w, bits, layout, n, d) == c).all()
    wv = oracle.pack(c, bits, "V")
    E = 32 // bits
    assert wv.shape == (-(-n // E), d)
    last = n % E
    if last:
        pad_mask = 0
        for e in range(last, E):
            pad_mask |= ((1 << bits) - 1) << oracle.code_bit_offset(e, bits)
        assert ((wv[-1].astype(np.uint64) & pad_mask) == 0).all()
    assert oracle.pack(c, bits, "K").shape == (d * bits // 32, n)


def test_batched_quantize_matches_units():
    x = kv_numpy(7, 0, ROLE_K, 2, 3, 40, 32, "float16")
    words, scale, minv, codes = oracle.quantize(x, 1, "K")
    assert words.shape == (2, 3, 1, 40)
    for b in range(2):
        for h in range(3):
            c, s, m, _ = oracle.quantize_unit(x[b, h], 1)
            assert (codes[b, h] == c).all() and (scale[b, h] == s).all() and (minv[b, h] == m).all()
            assert (words[b, h] == oracle.pack(c, 1, "K")).all()
    xv = kv_numpy(7, 0, ROLE_V, 1, 1, 33, 32, "float16")
    wv, *_ = oracle.quantize(xv, 2, "V")
    assert wv.shape == (1, 1, 3, 32)
