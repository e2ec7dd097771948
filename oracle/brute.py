"""Pure-Python brute force of the CalibQuant path, for tiny inputs.

TEST INFRASTRUCTURE (same import rule as ``oracle.cq_oracle``).  Written with
plain loops, exact fractions, ``math.fsum`` and ``math.exp`` so that it can be
checked by eye; it is deliberately formulated differently from the NumPy
oracle where the mathematics allows:

* codes come from an exhaustive nearest-grid-point search (QbitAI article on
  CalibQuant, section "Method", part 1: round a value in [mn, mx] to the
  nearest of the 2**b evenly spaced levels), ties going to the even level;
* attention is a loop over tokens with an explicit exp-sum.
"""
from __future__ import annotations

import math
from fractions import Fraction


def quantize_brute(x, bits):
    """x: list of n rows of d Python floats.  Returns (codes, mn, mx) with
    codes[i][j] the index k in 0..L of the level mn_j + k (mx_j - mn_j)/L nearest
    to x[i][j] (exact arithmetic; ties to even k)."""
    L = (1 << bits) - 1
    n, d = len(x), len(x[0])
    mn = [min(Fraction(x[i][j]) for i in range(n)) for j in range(d)]
    mx = [max(Fraction(x[i][j]) for i in range(n)) for j in range(d)]
    codes = [[0] * d for _ in range(n)]
    for j in range(d):
        if mx[j] == mn[j]:
            continue
        step = (mx[j] - mn[j]) / L
        for i in range(n):
            v = Fraction(x[i][j])
            best_k, best_err = None, None
            for k in range(L + 1):
                err = abs(v - (mn[j] + k * step))
                if best_err is None or err < best_err or (err == best_err and k % 2 == 0):
                    best_k, best_err = k, err
            codes[i][j] = best_k
    return codes, mn, mx


def quantize_brute_range(x, mn, mx, bits):
    """Codes of x (n rows of d Python floats) on a given range: codes[i][j] is
    the index k in 0..L of the level mn_j + k (mx_j - mn_j)/L nearest to
    x[i][j] (exact arithmetic, ties to even k), 0 when mx_j <= mn_j.  Values
    outside the range simply find an end level nearest."""
    L = (1 << bits) - 1
    n, d = len(x), len(x[0])
    codes = [[0] * d for _ in range(n)]
    for j in range(d):
        lo, hi = Fraction(mn[j]), Fraction(mx[j])
        if hi <= lo:
            continue
        step = (hi - lo) / L
        for i in range(n):
            v = Fraction(x[i][j])
            best_k, best_err = None, None
            for k in range(L + 1):
                err = abs(v - (lo + k * step))
                if best_err is None or err < best_err or (err == best_err and k % 2 == 0):
                    best_k, best_err = k, err
            codes[i][j] = best_k
    return codes


def decode_brute(q, Khat, Vhat, Kt, Vt, sm_scale, calib):
    """q: G lists of d; Khat/Vhat: n lists of d (already dequantized); Kt/Vt: T lists.

    calib: None or (a_lo, c_lo, a_hi, c_hi).  Returns G output lists.
    """
    G, d = len(q), len(q[0])
    out = []
    for g in range(G):
        vis = [sm_scale * math.fsum(q[g][j] * k[j] for j in range(d)) for k in Khat]
        if calib is not None and vis:
            a_lo, c_lo, a_hi, c_hi = calib
            m, M = min(vis), max(vis)
            lo, hi = a_lo * m + c_lo, a_hi * M + c_hi
            if M > m:
                vis = [lo + (s - m) * (hi - lo) / (M - m) for s in vis]
            else:
                vis = [lo for _ in vis]
        txt = [sm_scale * math.fsum(q[g][j] * k[j] for j in range(d)) for k in Kt]
        scores = vis + txt
        rows = list(Vhat) + list(Vt)
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        z = math.fsum(w)
        out.append([math.fsum(w[i] * rows[i][j] for i in range(len(rows))) / z for j in range(d)])
    return out
