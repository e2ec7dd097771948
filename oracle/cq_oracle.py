"""NumPy float64 reference of the CalibQuant visual-KV decode path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
(package ``extreme_bit_kv_amd``) never imports it and shares no code with it.

Sources, cited by page title and section:

[ART]  QbitAI article on CalibQuant, "在 InternVL-2.5 上达成 10 倍吞吐量提升"
       (abroadessay.com repost), section "Method" (要津/方法) with its three
       parts: (1) channel-wise KV-cache quantization, (2) post-scaling
       KV-cache management, (3) post-quantization calibration.
[ABS]  "CalibQuant: 1-Bit KV Cache Quantization for Multimodal LLMs",
       abstract (papers.pytorch.kr).
[REP]  Reportify summary of CalibQuant, "方法概述" (method overview).

All formulas were lost when the pages were extracted; every place where this
file has to pick a reading says so in a "Reading:" note.

Precision: inputs (float16 / float32) are promoted exactly; codes are decided
in exact integer arithmetic; everything else is float64.

Parity pins: every public function is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, brute force or textbook routines.
"""
from __future__ import annotations

from fractions import Fraction
from typing import NamedTuple, Optional, Tuple

import numpy as np


class Calib(NamedTuple):
    """Parameters of the calibration map g ([ART] Method part 3).

    Reading: the pages say g is linear and maps the interval [m, M] that holds
    the pre-softmax scores onto a target interval fixed by given parameters,
    but the parameters and the target interval were lost.  Both endpoints are
    taken as affine in the source endpoints:
        t_lo = a_lo * m + c_lo,   t_hi = a_hi * M + c_hi.
    (a, c) = (1, 0, 1, 0) is the identity; (tau_lo, 0, tau_hi, 0) is a relative
    interval; (0, t1, 0, t2) a fixed one.
    """
    a_lo: float
    c_lo: float
    a_hi: float
    c_hi: float


# --------------------------------------------------------------------------
# Exact representation of the inputs
# --------------------------------------------------------------------------

def exact_ints(x: np.ndarray) -> Tuple[np.ndarray, int]:
    """Return (X, k) with x == X * 2**-k exactly, X integral.

    float16 values are multiples of 2**-24 below 2**16 in magnitude, so X fits
    int64.  float32 values are multiples of 2**-149; X is then an object array
    of Python integers.
    """
    x = np.asarray(x)
    if x.dtype == np.float16:
        X = (x.astype(np.float64) * 2.0 ** 24).astype(np.int64)
        return X, 24
    if x.dtype == np.float32:
        flat = [int(Fraction(float(v)) * (1 << 149)) for v in x.ravel()]
        X = np.empty(x.size, dtype=object)
        X[:] = flat
        return X.reshape(x.shape), 149
    raise TypeError(f"inputs are float16 or float32, got {x.dtype}")


def nearest_f32(value: Fraction) -> np.float32:
    """float32 nearest to an exact rational, ties to even (IEEE RN)."""
    guess = np.float32(float(value))
    best = None
    for cand in (np.nextafter(guess, np.float32(-np.inf)), guess,
                 np.nextafter(guess, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        err = abs(Fraction(float(cand)) - value)
        even = (int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1) == 0
        key = (err, not even)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


# --------------------------------------------------------------------------
# Channel-wise quantization ([ART] Method part 1; [REP] method overview)
# --------------------------------------------------------------------------

def quantize_unit(x: np.ndarray, bits: int):
    """Channel-wise b-bit quantization of one head's cache block x[n, d].

    [ART] Method part 1: uniform integer quantization maps a value in a range
    to a discrete integer with a rounding operator; instead of global
    statistics the range is taken per channel (two d-vectors for a K block of
    n tokens and d channels), every row is quantized element-wise with them,
    and V is treated the same way.

    Readings:
      * range = per-channel [min, max] over the n tokens (the 1-bit codebook is
        said, in part 3, to always contain the minimum and the maximum);
      * code = round((x - mn) * L / (mx - mn)), L = 2**b - 1, with the rounding
        operator read as round-half-to-even of the exact real value;
      * a channel with mx == mn gets code 0 (any code reconstructs it exactly);
      * the stored parameters are scale = (mx - mn) / L (float32, correctly
        rounded from the exact quotient) and min = mn (exact in float32).

    Returns (codes int64 [n, d], scale float32 [d], minv float32 [d],
    scale_exact float64 [d]).
    """
    if bits not in (1, 2, 4, 8):
        raise ValueError("bits must be 1, 2, 4 or 8")
    x = np.asarray(x)
    n, d = x.shape
    L = (1 << bits) - 1
    if n == 0:
        z = np.zeros(d, np.float32)
        return np.zeros((0, d), np.int64), z, z.copy(), np.zeros(d)
    X, k = exact_ints(x)
    MN = X.min(axis=0)
    MX = X.max(axis=0)
    den = MX - MN
    live = den > 0
    den_safe = np.where(live, den, 1)
    num = (X - MN) * L
    q = num // den_safe
    r = num - q * den_safe
    up = (2 * r > den_safe) | ((2 * r == den_safe) & (q % 2 == 1))
    codes = np.where(live, q + up, 0).astype(np.int64)
    scale = np.empty(d, np.float32)
    scale_exact = np.empty(d, np.float64)
    for j in range(d):
        fr = Fraction(int(den[j]), L << k)
        scale[j] = nearest_f32(fr)
        scale_exact[j] = float(fr)
    minv = x.min(axis=0).astype(np.float32)
    return codes, scale, minv, scale_exact


# --------------------------------------------------------------------------
# Chunked prefill: the range gathered chunk by chunk, codes on a given range
# ([ART] Method part 1 applied to a visual segment that arrives in pieces)
# --------------------------------------------------------------------------

def range_update(mn, mx, x_chunk: np.ndarray, reset: bool):
    """Merge one chunk x_chunk[m, d] (m >= 1) of a unit's visual tokens into
    the running per-channel range (mn, mx), float32 [d].

    Reading: the range of [ART] Method part 1 is the per-channel minimum and
    maximum over the unit's tokens.  Minimum and maximum are associative, so
    a segment that arrives in chunks has, after its last chunk, exactly the
    range of the whole segment.  ``reset`` starts a new range from the chunk
    (mn and mx are then ignored).

    Returns (mn', mx', grew): grew is True when some channel's range became
    wider than (mn, mx) (always True under reset).
    """
    c = np.asarray(x_chunk)
    if c.ndim != 2 or c.shape[0] < 1:
        raise ValueError("a chunk is [m, d] with m >= 1")
    cmn = c.min(axis=0).astype(np.float32)
    cmx = c.max(axis=0).astype(np.float32)
    if reset:
        return cmn, cmx, True
    mn = np.asarray(mn, np.float32)
    mx = np.asarray(mx, np.float32)
    nmn = np.minimum(mn, cmn)
    nmx = np.maximum(mx, cmx)
    grew = bool(np.any(nmn < mn) or np.any(nmx > mx))
    return nmn, nmx, grew


def _exact_common(x: np.ndarray, mn: np.ndarray, mx: np.ndarray):
    """(X, MN, MX, k): x == X 2^-k, mn == MN 2^-k, mx == MX 2^-k exactly."""
    on_f16_grid = (x.dtype == np.float16 and
                   all(np.all(np.abs(v) <= 65504) and np.all(v.astype(np.float64) * 2.0 ** 24 ==
                                                          np.round(v.astype(np.float64) * 2.0 ** 24))
                       for v in (mn, mx)))
    if on_f16_grid:
        X, k = exact_ints(x)
        to = lambda v: (v.astype(np.float64) * 2.0 ** 24).astype(np.int64)   # noqa: E731
        return X, to(mn), to(mx), k
    X, k = exact_ints(x.astype(np.float32))           # float16 -> float32 is exact
    MN, _ = exact_ints(mn)
    MX, _ = exact_ints(mx)
    return X, MN, MX, k


def quantize_with_range(x: np.ndarray, mn, mx, bits: int):
    """Codes of one unit's block x[n, d] on the grid of a GIVEN per-channel
    range [mn, mx] (float32 [d]), for a chunked prefill in which the range is
    gathered before (or while) the codes are written.

    [ART] Method part 1's quantizer, with its range supplied instead of
    measured on x: code = round-half-to-even((x - mn) L / (mx - mn)), decided
    exactly, L = 2**b - 1.

    Readings:
      * a value outside [mn, mx] takes the nearest level, i.e. its code is
        clamped to [0, L] (with mn, mx the range of x itself no value is
        outside and this is ``quantize_unit``);
      * a channel with mx <= mn gets code 0 and scale 0;
      * stored parameters as in ``quantize_unit``: scale = (mx - mn)/L rounded
        to the nearest float32, min = mn.

    Returns (codes int64 [n, d], scale float32 [d], minv float32 [d]).
    """
    if bits not in (1, 2, 4, 8):
        raise ValueError("bits must be 1, 2, 4 or 8")
    x = np.asarray(x)
    mn = np.asarray(mn, np.float32)
    mx = np.asarray(mx, np.float32)
    n, d = x.shape
    L = (1 << bits) - 1
    X, MN, MX, k = _exact_common(x, mn, mx)
    den = MX - MN
    live = den > 0
    den_safe = np.where(live, den, 1)
    num = (X - MN) * L
    q = num // den_safe                                   # floor, also for negative num
    r = num - q * den_safe                                # 0 <= r < den
    up = (2 * r > den_safe) | ((2 * r == den_safe) & (q % 2 != 0))
    codes = np.clip(np.where(live, q + up, 0).astype(np.int64), 0, L)
    scale = np.zeros(d, np.float32)
    for j in range(d):
        if live[j]:
            scale[j] = nearest_f32(Fraction(int(den[j]), L << k))
    return codes.reshape(n, d), scale, mn.copy()


def dequant(codes: np.ndarray, scale: np.ndarray, minv: np.ndarray) -> np.ndarray:
    """x_hat = min + code * scale, per channel ([ART] Method part 2)."""
    return np.asarray(minv, np.float64) + np.asarray(codes, np.float64) * np.asarray(scale, np.float64)


# --------------------------------------------------------------------------
# Packed layouts (not on the pages: the storage format of this library)
# --------------------------------------------------------------------------

def code_bit_offset(e: int, bits: int) -> int:
    """Bit offset of element e (0 <= e < 32/bits) inside a 32-bit word.

    Element e sits in byte (e mod 4) at sub-offset bits * floor(e / 4), so that
    (word >> (bits*s)) & (L * 0x01010101) yields elements 4s .. 4s+3 in bytes
    0 .. 3.
    """
    return 8 * (e % 4) + bits * (e // 4)


def pack(codes: np.ndarray, bits: int, layout: str) -> np.ndarray:
    """Pack one unit's codes[n, d] into uint32 words.

    layout "K": words[W][n], W = d*bits/32; word (w, i) holds channels
                w*E .. w*E+E-1 of token i (E = 32/bits).
    layout "V": words[R][d], R = ceil(n/E); word (r, j) holds tokens
                r*E .. r*E+E-1 of channel j; elements past token n-1 are 0.
    """
    codes = np.asarray(codes, np.int64)
    n, d = codes.shape
    E = 32 // bits
    L = (1 << bits) - 1
    assert codes.min(initial=0) >= 0 and codes.max(initial=0) <= L
    if layout == "K":
        assert d % E == 0
        words = np.zeros((d // E, n), np.uint64)
        for w in range(d // E):
            for e in range(E):
                words[w] |= codes[:, w * E + e].astype(np.uint64) << np.uint64(code_bit_offset(e, bits))
    elif layout == "V":
        R = -(-n // E)
        padded = np.zeros((R * E, d), np.int64)
        padded[:n] = codes
        words = np.zeros((R, d), np.uint64)
        for e in range(E):
            words |= padded[e::E].astype(np.uint64) << np.uint64(code_bit_offset(e, bits))
    else:
        raise ValueError(layout)
    return words.astype(np.uint32)


def unpack(words: np.ndarray, bits: int, layout: str, n: int, d: int) -> np.ndarray:
    """Inverse of :func:`pack`."""
    words = np.asarray(words, np.uint64)
    E = 32 // bits
    L = np.uint64((1 << bits) - 1)
    if layout == "K":
        codes = np.zeros((n, d), np.int64)
        for w in range(d // E):
            for e in range(E):
                codes[:, w * E + e] = (words[w] >> np.uint64(code_bit_offset(e, bits))) & L
    elif layout == "V":
        R = -(-n // E)
        full = np.zeros((R * E, d), np.int64)
        for e in range(E):
            full[e::E] = (words >> np.uint64(code_bit_offset(e, bits))) & L
        codes = full[:n]
    else:
        raise ValueError(layout)
    return codes


# --------------------------------------------------------------------------
# Calibration ([ART] Method part 3; [REP] method overview)
# --------------------------------------------------------------------------

def calibrate_rows(s: np.ndarray, calib: Calib):
    """Apply g row by row to pre-softmax scores s[R, n].

    [ART] Method part 3: 1-bit dequantized values pile up at the extremes,
    which distorts attention scores; a linear map g, applied to the scores
    before softmax, sends the interval [m, M] holding them onto a target
    interval.  [REP] calls it a linear transform that adjusts the peaks of the
    pre-softmax scores.

    Readings: m, M are the min and max of each row (one query head); the
    target interval is [t_lo, t_hi] as in :class:`Calib`; a row with M == m
    maps to t_lo.

    Returns (calibrated scores, m, M).
    """
    s = np.asarray(s, np.float64)
    m = s.min(axis=-1, keepdims=True)
    M = s.max(axis=-1, keepdims=True)
    t_lo = calib.a_lo * m + calib.c_lo
    t_hi = calib.a_hi * M + calib.c_hi
    span = M - m
    live = span > 0
    out = np.where(live, t_lo + (s - m) * (t_hi - t_lo) / np.where(live, span, 1.0), t_lo)
    return out, m[..., 0], M[..., 0]


# --------------------------------------------------------------------------
# Decode attention
# --------------------------------------------------------------------------

def _softmax_rows(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def dense_scores(q, K, sm_scale):
    """Textbook pre-softmax scores sm_scale * q . k_i of q[G, d] over K[N, d] -> [G, N]."""
    return sm_scale * (np.asarray(q, np.float64) @ np.asarray(K, np.float64).T)


def attend_dense(q, K, V, sm_scale):
    """Textbook softmax attention for one kv head: q[G, d], K[N, d], V[N, d]."""
    return _softmax_rows(dense_scores(q, K, sm_scale)) @ np.asarray(V, np.float64)


def visual_scores(q, k_codes, k_scale, k_min, sm_scale: float):
    """Pre-softmax visual scores s_i = sm_scale * q . k_hat_i of G query heads
    q[G, d] over one kv head's quantized keys, explicit-dequantization form
    ([ART] Method part 2: k_hat_i = min_K + c_i * scale_K).  Returns [G, n]."""
    q = np.asarray(q, np.float64)
    return sm_scale * (q @ dequant(k_codes, k_scale, k_min).T)


def decode_unit(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min,
                k_tail, v_tail, sm_scale: float, calib: Optional[Calib]):
    """Decode attention of G query heads q[G, d] over one kv head.

    Explicit-dequantization form: the quantized visual keys and values are
    reconstructed ([ART] Method part 2), visual scores are
    s_i = sm_scale * q . k_hat_i, calibrated by g when ``calib`` is given
    ([ART] Method part 3), text-tail scores (the tail stays in full precision:
    only the visual cache is quantized, [ART] introduction, [ABS]) are
    sm_scale * q . kt_j, and one softmax runs over both.

    Readings: g acts on the scaled logits, per query head, over the visual
    tokens only (the distortion it corrects comes from quantized keys).
    """
    q = np.asarray(q, np.float64)
    n = np.asarray(k_codes).shape[0]
    T = 0 if k_tail is None else np.asarray(k_tail).shape[0]
    if n + T == 0:
        raise ValueError("no tokens to attend over")
    parts_s, parts_v = [], []
    if n:
        Vh = dequant(v_codes, v_scale, v_min)
        s = visual_scores(q, k_codes, k_scale, k_min, sm_scale)
        if calib is not None:
            s, _, _ = calibrate_rows(s, calib)
        parts_s.append(s)
        parts_v.append(Vh)
    if T:
        parts_s.append(sm_scale * (q @ np.asarray(k_tail, np.float64).T))
        parts_v.append(np.asarray(v_tail, np.float64))
    p = _softmax_rows(np.concatenate(parts_s, axis=-1))
    return p @ np.concatenate(parts_v, axis=0)


def decode_unit_postscaled(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min,
                           k_tail, v_tail, sm_scale: float, calib: Optional[Calib]):
    """The same result computed from the integer codes with deferred scaling.

    [ART] Method part 2 (and [REP]): the per-channel dequantization is moved
    into the following vector products, so only the integer codes take part
    in them:  s_i = sm_scale * ((q * scale_K) . c_i + q . min_K)  and
    o = scale_V * sum_i p_i c_i + (sum_i p_i) * min_V + sum_j p_j vt_j.
    The min_V term is weighted by the visual probability mass, which is 1 only
    when there is no text tail.
    """
    q = np.asarray(q, np.float64)
    n = np.asarray(k_codes).shape[0]
    T = 0 if k_tail is None else np.asarray(k_tail).shape[0]
    if n + T == 0:
        raise ValueError("no tokens to attend over")
    parts = []
    if n:
        kc = np.asarray(k_codes, np.float64)
        s = sm_scale * ((q * np.asarray(k_scale, np.float64)) @ kc.T
                        + (q @ np.asarray(k_min, np.float64))[:, None])
        if calib is not None:
            s, _, _ = calibrate_rows(s, calib)
        parts.append(s)
    if T:
        parts.append(sm_scale * (q @ np.asarray(k_tail, np.float64).T))
    p = _softmax_rows(np.concatenate(parts, axis=-1))
    o = np.zeros_like(q)
    if n:
        pv = p[:, :n]
        o += np.asarray(v_scale, np.float64) * (pv @ np.asarray(v_codes, np.float64))
        o += pv.sum(axis=-1, keepdims=True) * np.asarray(v_min, np.float64)
    if T:
        o += p[:, n:] @ np.asarray(v_tail, np.float64)
    return o


# --------------------------------------------------------------------------
# Batched drivers over (batch, kv head)
# --------------------------------------------------------------------------

def quantize(x: np.ndarray, bits: int, layout: str):
    """x[B, H, n, d] -> (words, scale[B, H, d], minv[B, H, d], codes[B, H, n, d])."""
    B, H, n, d = x.shape
    words, scales, mins, codes = [], [], [], []
    for b in range(B):
        for h in range(H):
            c, sc, mn, _ = quantize_unit(x[b, h], bits)
            codes.append(c)
            words.append(pack(c, bits, layout))
            scales.append(sc)
            mins.append(mn)
    shp = words[0].shape
    return (np.stack(words).reshape(B, H, *shp), np.stack(scales).reshape(B, H, d),
            np.stack(mins).reshape(B, H, d), np.stack(codes).reshape(B, H, n, d))


def decode_attn(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min,
                k_tail, v_tail, sm_scale: float, calib: Optional[Calib]):
    """q[B, Hq, d]; codes[B, Hkv, n, d]; params[B, Hkv, d]; tails[B, Hkv, T, d] or None.

    Query head hq reads kv head hq // (Hq / Hkv).
    """
    B, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hkv):
            kt = None if k_tail is None else k_tail[b, h]
            vt = None if v_tail is None else v_tail[b, h]
            out[b, h * G:(h + 1) * G] = decode_unit(
                q[b, h * G:(h + 1) * G], k_codes[b, h], k_scale[b, h], k_min[b, h],
                v_codes[b, h], v_scale[b, h], v_min[b, h], kt, vt, sm_scale, calib)
    return out
