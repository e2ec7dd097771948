"""Pins of the oracle's decode attention and calibration (no GPU).

Pages: QbitAI article on CalibQuant, section "Method" part 2 (post-scaling:
the per-channel dequantization is deferred into the following vector
products, so the result is that of dequantize-then-attend) and part 3
(calibration: a linear map g sends the score interval [m, M] onto a target
interval before softmax).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import Calib
from workloads import ROLE_K, ROLE_KTAIL, ROLE_V, ROLE_VTAIL, kv_numpy, q_numpy

SM = 1.0 / np.sqrt(128.0)
RELATIVE = Calib(0.9, 0.0, 0.8, 0.0)
ABSOLUTE = Calib(0.0, -4.0, 0.0, 4.0)
IDENTITY = Calib(1.0, 0.0, 1.0, 0.0)


def _unit(n, T, d=128, bits=1, seed=3, G=4):
    x_k = kv_numpy(seed, 0, ROLE_K, 1, 1, n, d)[0, 0]
    x_v = kv_numpy(seed, 0, ROLE_V, 1, 1, n, d)[0, 0]
    kc, ks, km, _ = oracle.quantize_unit(x_k, bits)
    vc, vs, vm, _ = oracle.quantize_unit(x_v, bits)
    kt = kv_numpy(seed, 0, ROLE_KTAIL, 1, 1, T, d)[0, 0] if T else None
    vt = kv_numpy(seed, 0, ROLE_VTAIL, 1, 1, T, d)[0, 0] if T else None
    q = q_numpy(seed, 0, 1, G, d)[0]
    return q, kc, ks, km, vc, vs, vm, kt, vt


# ---- P5: post-scaled form equals explicit dequantization --------------------

@pytest.mark.parametrize("T", [0, 16])
@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE])
@pytest.mark.parametrize("bits", [1, 4])
def test_postscaled_equals_dequant(T, calib, bits):
    args = _unit(96, T, bits=bits)
    a = oracle.decode_unit(*args, SM, calib)
    b = oracle.decode_unit_postscaled(*args, SM, calib)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))


# ---- P6: calibration map -------------------------------------------------

def test_calibration_endpoints_and_linearity():
    rng = np.random.default_rng(0)
    s = rng.standard_normal((5, 33)) * 3
    for c in (RELATIVE, ABSOLUTE, Calib(0.5, 1.0, -1.0, 2.0)):
        out, m, M = oracle.calibrate_rows(s, c)
        assert np.allclose(m, s.min(-1), rtol=0, atol=0) and np.allclose(M, s.max(-1), rtol=0, atol=0)
        lo, hi = c.a_lo * m + c.c_lo, c.a_hi * M + c.c_hi
        idx_lo, idx_hi = s.argmin(-1), s.argmax(-1)
        r = np.arange(5)
        assert np.allclose(out[r, idx_lo], lo, rtol=1e-15, atol=1e-14)
        assert np.allclose(out[r, idx_hi], hi, rtol=1e-15, atol=1e-14)
        # affine: midpoint maps to midpoint
        mid = (s[:, :1] + s[:, 1:2]) / 2
        g_mid = lo[:, None] + (mid - m[:, None]) * ((hi - lo) / (M - m))[:, None]
        assert np.allclose((out[:, :1] + out[:, 1:2]) / 2, g_mid, rtol=1e-14, atol=1e-13)
    out, _, _ = oracle.calibrate_rows(s, IDENTITY)
    assert np.allclose(out, s, rtol=1e-15, atol=1e-14)


def test_calibration_constant_row():
    s = np.full((2, 7), 1.5)
    out, m, M = oracle.calibrate_rows(s, RELATIVE)
    assert (out == 0.9 * 1.5).all()


def test_identity_calibration_is_no_op():
    args = _unit(64, 8)
    assert np.allclose(oracle.decode_unit(*args, SM, IDENTITY), oracle.decode_unit(*args, SM, None),
                       rtol=1e-13, atol=1e-13)


def test_calibration_is_a_temperature_without_tail():
    """With no tail, softmax(g(s)) = softmax(lambda * s), lambda = (t_hi - t_lo)/(M - m):
    the calibrated output equals textbook attention with the query scaled by lambda."""
    q, kc, ks, km, vc, vs, vm, _, _ = _unit(80, 0)
    Kh, Vh = oracle.dequant(kc, ks, km), oracle.dequant(vc, vs, vm)
    out = oracle.decode_unit(q, kc, ks, km, vc, vs, vm, None, None, SM, RELATIVE)
    s = SM * (q.astype(np.float64) @ Kh.T)
    m, M = s.min(-1), s.max(-1)
    lam = ((RELATIVE.a_hi * M + RELATIVE.c_hi) - (RELATIVE.a_lo * m + RELATIVE.c_lo)) / (M - m)
    for g in range(q.shape[0]):
        ref = oracle.attend_dense(lam[g] * q[g:g + 1].astype(np.float64), Kh, Vh, SM)
        assert np.allclose(out[g], ref[0], rtol=1e-12, atol=1e-12)


# ---- P7: lossless special cases reduce to textbook attention ----------------

def _two_level(n, d, rng):
    lo = rng.standard_normal(d).astype(np.float16)
    hi = (lo.astype(np.float32) + rng.uniform(0.5, 3, d)).astype(np.float16)
    pick = rng.integers(0, 2, (n, d))
    pick[0], pick[1] = 0, 1
    return np.where(pick == 1, hi, lo).astype(np.float16)


def _grid256(n, d, rng):
    base = rng.integers(-8, 8, d) * 0.25
    step = 2.0 ** rng.integers(-6, -3, d)
    k = rng.integers(0, 256, (n, d))
    k[0], k[1] = 0, 255
    return (base + k * step).astype(np.float16)


@pytest.mark.parametrize("bits,maker", [(1, _two_level), (8, _grid256)])
@pytest.mark.parametrize("T", [0, 8])
def test_lossless_cases_equal_sdpa(bits, maker, T):
    rng = np.random.default_rng(bits + T)
    n, d, G = 50, 128, 4
    K, V = maker(n, d, rng), maker(n, d, rng)
    kc, ks, km, _ = oracle.quantize_unit(K, bits)
    vc, vs, vm, _ = oracle.quantize_unit(V, bits)
    assert np.array_equal(oracle.dequant(kc, ks, km), K.astype(np.float64))
    assert np.array_equal(oracle.dequant(vc, vs, vm), V.astype(np.float64))
    q = rng.standard_normal((G, d)).astype(np.float16)
    kt = rng.standard_normal((T, d)).astype(np.float16) if T else None
    vt = rng.standard_normal((T, d)).astype(np.float16) if T else None
    out = oracle.decode_unit(q, kc, ks, km, vc, vs, vm, kt, vt, SM, None)
    Kall = K if not T else np.concatenate([K, kt])
    Vall = V if not T else np.concatenate([V, vt])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q, dtype=torch.float64)[None, :, None, :],
        torch.tensor(Kall, dtype=torch.float64)[None, None].expand(1, G, -1, -1),
        torch.tensor(Vall, dtype=torch.float64)[None, None].expand(1, G, -1, -1),
        scale=SM)[0, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


# ---- P8: degenerate closed forms -------------------------------------------

def test_single_token_returns_its_value():
    q, kc, ks, km, vc, vs, vm, _, _ = _unit(1, 0)
    out = oracle.decode_unit(q, kc, ks, km, vc, vs, vm, None, None, SM, RELATIVE)
    assert np.allclose(out, np.broadcast_to(oracle.dequant(vc, vs, vm)[0], out.shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("calib", [None, RELATIVE])
def test_zero_query_averages_values(calib):
    _, kc, ks, km, vc, vs, vm, _, _ = _unit(37, 0)
    q = np.zeros((4, 128), np.float16)
    out = oracle.decode_unit(q, kc, ks, km, vc, vs, vm, None, None, SM, calib)
    mean = oracle.dequant(vc, vs, vm).mean(axis=0)
    assert np.allclose(out, np.broadcast_to(mean, out.shape), rtol=1e-13, atol=1e-13)


def test_tail_only():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 128)).astype(np.float16)
    kt = rng.standard_normal((5, 128)).astype(np.float16)
    vt = rng.standard_normal((5, 128)).astype(np.float16)
    empty = np.zeros((0, 128), np.int64)
    z = np.zeros(128, np.float32)
    out = oracle.decode_unit(q, empty, z, z, empty, z, z, kt, vt, SM, RELATIVE)
    assert np.allclose(out, oracle.attend_dense(q, kt, vt, SM), rtol=1e-13, atol=1e-13)


# ---- P9: brute force agrees with the NumPy oracle ---------------------------

@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE])
@pytest.mark.parametrize("T", [0, 3])
def test_brute_force_decode(calib, T):
    rng = np.random.default_rng(T)
    n, d, G, bits = 8, 8, 2, 2
    K = rng.standard_normal((n, d)).astype(np.float16)
    V = rng.standard_normal((n, d)).astype(np.float16)
    kc, ks, km, _ = oracle.quantize_unit(K, bits)
    vc, vs, vm, _ = oracle.quantize_unit(V, bits)
    bk, _, _ = oracle.quantize_brute(K.astype(np.float64).tolist(), bits)
    assert kc.tolist() == bk
    q = rng.standard_normal((G, d)).astype(np.float16)
    kt = rng.standard_normal((T, d)).astype(np.float16) if T else None
    vt = rng.standard_normal((T, d)).astype(np.float16) if T else None
    sm = 0.37
    out = oracle.decode_unit(q, kc, ks, km, vc, vs, vm, kt, vt, sm, calib)
    ref = oracle.decode_brute(
        q.astype(np.float64).tolist(), oracle.dequant(kc, ks, km).tolist(),
        oracle.dequant(vc, vs, vm).tolist(),
        [] if kt is None else kt.astype(np.float64).tolist(),
        [] if vt is None else vt.astype(np.float64).tolist(), sm, calib)
    assert np.allclose(out, np.array(ref), rtol=1e-12, atol=1e-12)


def test_brute_force_tiny_config_unit():
    """The fp32 single-head workload: codes from brute force equal the oracle's."""
    x = kv_numpy(1, 0, ROLE_K, 1, 1, 256, 128, "float32")[0, 0]
    codes, *_ = oracle.quantize_unit(x[:, :16], 1)
    ref, _, _ = oracle.quantize_brute(x[:, :16].astype(np.float64).tolist(), 1)
    assert codes.tolist() == ref


# ---- P10: invariances --------------------------------------------------------

def test_gqa_equals_replicated_single_heads():
    B, Hkv, G, n, T, d = 1, 2, 4, 24, 4, 128
    x_k = kv_numpy(5, 0, ROLE_K, B, Hkv, n, d)
    x_v = kv_numpy(5, 0, ROLE_V, B, Hkv, n, d)
    _, ks, km, kc = oracle.quantize(x_k, 1, "K")
    _, vs, vm, vc = oracle.quantize(x_v, 1, "V")
    kt = kv_numpy(5, 0, ROLE_KTAIL, B, Hkv, T, d)
    vt = kv_numpy(5, 0, ROLE_VTAIL, B, Hkv, T, d)
    q = q_numpy(5, 0, B, Hkv * G, d)
    out = oracle.decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, SM, RELATIVE)
    for hq in range(Hkv * G):
        h = hq // G
        one = oracle.decode_unit(q[0, hq:hq + 1], kc[0, h], ks[0, h], km[0, h], vc[0, h], vs[0, h],
                                 vm[0, h], kt[0, h], vt[0, h], SM, RELATIVE)
        assert np.allclose(out[0, hq], one[0], rtol=1e-14, atol=1e-14)


def test_token_permutation_invariance():
    q, kc, ks, km, vc, vs, vm, kt, vt = _unit(40, 6)
    perm = np.random.default_rng(1).permutation(40)
    tp = np.random.default_rng(2).permutation(6)
    a = oracle.decode_unit(q, kc, ks, km, vc, vs, vm, kt, vt, SM, RELATIVE)
    b = oracle.decode_unit(q, kc[perm], ks, km, vc[perm], vs, vm, kt[tp], vt[tp], SM, RELATIVE)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
