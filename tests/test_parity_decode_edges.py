"""GPU decode attention vs the oracle on the method's degenerate and
numerically hard cases, on every decode schedule.

The calibration map g (QbitAI article on CalibQuant, "Method" part 3) sends
the score interval [m, M] of each query head onto [t_lo, t_hi]; the cases
below reach its degenerate interval (M == m), its reversed target
(t_hi < t_lo), a narrow score range on a large common offset, many identical
visual tokens whose weight sits far below the dominant token's, and a text
tail token that dominates the softmax ("Method" part 2 for the post-scaled
products; only the visual cache is quantized, per the abstract).  Outputs must
be within 2e-3 of the oracle (inf-norm per head vector) on every path that
takes the shape.
"""
import functools

import numpy as np
import pytest

import oracle
from helpers import REL_TOL, calib_f32, note, rel_err

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")

SM = 1.0 / np.sqrt(128.0)
D = 128
RELATIVE = (0.9, 0.0, 0.8, 0.0)
ABSOLUTE = (0.0, -4.0, 0.0, 4.0)
WIDE = (0.0, -10.0, 0.0, 10.0)          # exp(t_lo - t_hi) far below the 2^-22 grid of older kernels
REVERSED = (0.5, 1.0, -1.0, 2.0)       # t_hi < t_lo on positive scores
REVERSED_REL = (1.0, 0.0, 0.5, 0.0)    # t_hi = M/2 < t_lo = m on scores in [m, M], 0 < m, M < 2m
IDENTITY = (1.0, 0.0, 1.0, 0.0)

P = cqb
B1_PATHS = [P.CQ_PATH_GENERIC, P.CQ_PATH_AUTO, P.CQ_PATH_FAST_ONE, P.CQ_PATH_FAST_LDS, P.CQ_PATH_FAST_PIPE,
            P.CQ_PATH_FAST_SPLIT, P.CQ_PATH_FAST_WIDE]
BN_PATHS = [P.CQ_PATH_GENERIC, P.CQ_PATH_AUTO, P.CQ_PATH_FAST_ONE]


# --------------------------------------------------------------------------
# inputs (host, float16), each family seeded
# --------------------------------------------------------------------------

def _rng(*key):
    return np.random.default_rng([2024, *key])


def _h(a):
    return np.asarray(a, np.float64).astype(np.float16)


def _base(key, B, Hkv, G, n, T, kmean=0.0, kstd=1.0, qpos=False):
    r = _rng(*key)
    K = _h(kmean + kstd * r.normal(size=(B, Hkv, n, D)))
    V = _h(r.normal(size=(B, Hkv, n, D)) * r.uniform(0.5, 2.0, size=(1, 1, 1, D)))
    q = r.normal(size=(B, Hkv * G, D))
    q = _h(np.abs(q) if qpos else q)
    kt = _h(r.normal(size=(B, Hkv, T, D))) if T else None
    vt = _h(r.normal(size=(B, Hkv, T, D))) if T else None
    return K, V, q, kt, vt


@functools.lru_cache(maxsize=None)
def case(name, n, T):
    """(K, V, q, kt, vt) of one named family; B = 2, 2 kv heads, G = 4 unless noted."""
    B, Hkv, G = 2, 2, 4
    if name == "q_zero":                       # every score equal: M == m
        K, V, q, kt, vt = _base((1, n, T), B, Hkv, G, n, T)
        q = np.zeros_like(q)
    elif name == "same_tokens":                # identical visual keys: M == m
        K, V, q, kt, vt = _base((2, n, T), B, Hkv, G, n, T)
        K = np.ascontiguousarray(np.broadcast_to(K[:, :, :1], K.shape))
    elif name == "positive":                   # scores in [m, M] with 0 < m < M < 2m
        K, V, q, kt, vt = _base((3, n, T), B, Hkv, G, n, T, kmean=5.0, qpos=True)
    elif name == "offset":                     # channel means far above their spread
        K, V, q, kt, vt = _base((4, n, T), B, Hkv, G, n, T, kmean=100.0, kstd=0.5)
    elif name == "tail_dominant":              # one text token far above every visual score
        K, V, q, kt, vt = _base((5, n, T), B, Hkv, G, n, T)
        for b in range(B):
            for h in range(Hkv):
                qs = q[b, h * G:(h + 1) * G].astype(np.float64)
                u = qs.sum(0) / np.linalg.norm(qs.sum(0))
                kt[b, h, T // 2] = _h(u * 45.0 / SM / max(1e-3, float((qs @ u).min())))
    else:
        raise ValueError(name)
    return K, V, q, kt, vt


@functools.lru_cache(maxsize=None)
def duplicates(n, T, ratios):
    """n - 1 identical visual tokens and one dominant token (token 0); per query
    head the weight of a duplicate relative to the dominant token is about
    ratios[h] (the keys are two-valued per channel, so 1-bit codes hold them
    exactly and the gap of the scores is sm_scale q . (k_dom - k_dup))."""
    r = _rng(6, n, T)
    G = len(ratios)
    k_dup = r.normal(size=D)
    delta = np.where(r.random(D) < 0.5, -1.0, 1.0) * r.uniform(0.5, 1.5, size=D)
    k_dom = k_dup + delta
    K = np.empty((1, 1, n, D))
    K[:] = k_dup
    K[0, 0, 0] = k_dom
    K = _h(K)
    dk = K[0, 0, 0].astype(np.float64) - K[0, 0, 1].astype(np.float64)
    V = np.empty((1, 1, n, D))
    V[:] = r.normal(size=D) * 3.0
    V[0, 0, 0] = r.normal(size=D) * 3.0
    V = _h(V)
    base = r.normal(size=D) * 0.05
    base -= dk * (base @ dk) / (dk @ dk)            # no effect on the gap
    q = np.stack([base + dk * (-np.log(rt) / SM) / (dk @ dk) for rt in ratios])[None]
    q = _h(q)
    kt = _h(r.normal(size=(1, 1, T, D)) * 0.1) if T else None
    vt = _h(r.normal(size=(1, 1, T, D))) if T else None
    return K, V, q, kt, vt


# --------------------------------------------------------------------------
# run and compare
# --------------------------------------------------------------------------

def _dev(a):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _takes(path, bits, G, n, T):
    """Whether a forced path takes the shape (else the library returns CQ_ERR_UNSUPPORTED)."""
    fast = G in (1, 2, 4) and n % 32 == 0
    if path == P.CQ_PATH_FAST_ONE:
        return fast
    if path == P.CQ_PATH_FAST_SPLIT:
        return fast and bits == 1 and n > 0 and T <= 256
    if path == P.CQ_PATH_FAST_LDS:
        return fast and bits == 1 and G * -(-n // 128) <= 256 and T <= 256
    if path == P.CQ_PATH_FAST_PIPE:
        return fast and bits == 1 and 32 <= n <= 8192 and T <= 128
    if path == P.CQ_PATH_FAST_WIDE:
        return fast and bits == 1 and n <= 4096 and T <= 256
    return True


def _oracle_all(K, V, q, kt, vt, bits, calib):
    B, Hkv, n, _ = K.shape
    G = q.shape[1] // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hkv):
            kc, ks, km, _ = oracle.quantize_unit(K[b, h], bits)
            vc, vs, vm, _ = oracle.quantize_unit(V[b, h], bits)
            out[b, h * G:(h + 1) * G] = oracle.decode_unit(
                q[b, h * G:(h + 1) * G], kc, ks, km, vc, vs, vm,
                None if kt is None else kt[b, h], None if vt is None else vt[b, h], SM, calib_f32(calib))
    return out


def _check(inputs, bits, calib, paths, label):
    import torch
    K, V, q, kt, vt = inputs
    B, Hkv, n, _ = K.shape
    G = q.shape[1] // Hkv
    T = 0 if kt is None else kt.shape[2]
    ref = _oracle_all(K, V, q, kt, vt, bits, calib)
    assert np.all(np.isfinite(ref))
    dK, dV, dq, dkt, dvt = (_dev(a) for a in (K, V, q, kt, vt))
    kc, ks, km = cqb.cq_quantize_kv(dK, bits, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(dV, bits, cqb.CQ_LAYOUT_V)
    checked = 0
    for path in paths:
        note(f"decode edge {label} n={n} T={T} bits={bits} calib={calib} path={path}")
        if not _takes(path, bits, G, n, T):
            with pytest.raises(cqb.CQError) as ei:
                cqb.cq_decode_attn(dq, kc, ks, km, vc, vs, vm, dkt, dvt, n=n, bits=bits, sm_scale=SM,
                                   calib=calib, path=path)
            assert ei.value.status == 2             # CQ_ERR_UNSUPPORTED
            continue
        out = cqb.cq_decode_attn(dq, kc, ks, km, vc, vs, vm, dkt, dvt, n=n, bits=bits, sm_scale=SM,
                                 calib=calib, path=path, out_dtype=torch.float32)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got)), f"path {path}: non-finite output"
        err = rel_err(got, ref)
        assert err <= REL_TOL, f"path {path}: relative error {err:.3e} > {REL_TOL}"
        checked += 1
    assert checked > 0


@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE, WIDE, REVERSED])
@pytest.mark.parametrize("T", [0, 16])
@pytest.mark.parametrize("name", ["q_zero", "same_tokens"])
def test_degenerate_interval(name, T, calib):
    """M == m: g sends every visual score to t_lo, so the visual weights are
    uniform; with a wide target the visual maximum is t_lo, not max(t_lo, t_hi)."""
    _check(case(name, 800, T), 1, calib, B1_PATHS, name)


@pytest.mark.parametrize("calib", [REVERSED, REVERSED_REL, RELATIVE, WIDE])
@pytest.mark.parametrize("T", [0, 64])
def test_reversed_target(T, calib):
    """Positive scores: (1, 0, 0.5, 0) and (0.5, 1, -1, 2) give t_hi < t_lo,
    a decreasing g whose largest value is t_lo."""
    _check(case("positive", 1056, T), 1, calib, B1_PATHS, "positive")


@pytest.mark.parametrize("calib", [ABSOLUTE, WIDE, RELATIVE, None])
@pytest.mark.parametrize("T", [0, 64])
def test_narrow_range_large_offset(T, calib):
    """Key channels with mean 100 and spread 0.5: the scores share a large
    common offset (q . min_K) and g stretches their narrow range."""
    _check(case("offset", 1056, T), 1, calib, B1_PATHS, "offset")


@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE])
def test_tail_token_dominates(calib):
    _check(case("tail_dominant", 1056, 64), 1, calib, B1_PATHS, "tail_dominant")


RATIOS = (1.4 * 2.0 ** -22, 2.0 ** -20, 0.6 * 2.0 ** -22, 1e-3)


@pytest.mark.parametrize("n", [8192, 32768])
@pytest.mark.parametrize("T", [0, 16])
@pytest.mark.parametrize("calib", [None, IDENTITY])
def test_duplicated_tokens_near_the_weight_floor(n, T, calib):
    """n - 1 identical visual tokens whose weights sit near 2^-22 of the
    dominant token's: their rounding errors do not cancel, so their total must
    still be right."""
    _check(duplicates(n, T, RATIOS), 1, calib, B1_PATHS, "duplicates")


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("calib", [None, RELATIVE, WIDE])
@pytest.mark.parametrize("name", ["q_zero", "same_tokens", "offset", "tail_dominant"])
def test_multibit_edges(bits, calib, name):
    _check(case(name, 1056, 64), bits, calib, BN_PATHS, name)


@pytest.mark.parametrize("n", [8192, 32768])
@pytest.mark.parametrize("bits", [2, 4, 8])
def test_multibit_duplicates(bits, n):
    _check(duplicates(n, 16, RATIOS), bits, None, BN_PATHS, "duplicates")
