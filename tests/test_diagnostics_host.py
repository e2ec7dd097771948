"""Host statistics of the score-distribution diagnostic (no GPU): closed forms."""
import math

import numpy as np
import pytest

diag = pytest.importorskip("extreme_bit_kv_amd.diagnostics")


def test_kl_closed_form_and_invariances():
    s = np.array([[0.0, 0.0], [1.0, -2.0]])
    r = np.array([[0.0, math.log(3.0)], [1.0, -2.0]])
    kl = diag.kl_rows(s, r)
    # p = (1/2, 1/2), q = (1/4, 3/4)
    assert kl[0] == pytest.approx(0.5 * math.log(2.0) + 0.5 * math.log(2.0 / 3.0), rel=1e-12)
    assert kl[1] == pytest.approx(0.0, abs=1e-15)
    # softmax is shift invariant, KL(p || p) = 0, KL >= 0
    rng = np.random.default_rng(0)
    a = rng.standard_normal((5, 40)) * 3
    b = rng.standard_normal((5, 40)) * 3
    assert np.allclose(diag.kl_rows(a, a + 7.0), 0.0, atol=1e-12)
    assert (diag.kl_rows(a, b) >= 0).all()


def test_histogram_and_tv():
    edges = np.linspace(0.0, 4.0, 5)
    h = diag.histogram(np.array([0.5, 1.5, 1.6, 3.9, 100.0]), edges)   # 100 clips into the last bin
    assert np.allclose(h, [0.2, 0.4, 0.0, 0.4]) and h.sum() == pytest.approx(1.0)
    assert diag.tv_distance(h, h) == 0.0
    assert diag.tv_distance([1.0, 0.0], [0.0, 1.0]) == 1.0


def test_default_sweep_and_report_format():
    cs = list(diag.default_calibs())
    assert (1.0, 0.0, 1.0, 0.0) not in cs and len(cs) == 13
    res = {"bits": 1, "shape": [1, 4, 1, 8], "settings": [
        {"calib": None, "kl_mean": 0.1, "kl_median": 0.05, "tv": 0.2, "mae": 0.3},
        {"calib": (0.9, 0.0, 0.8, 0.0), "kl_mean": 0.05, "kl_median": 0.02, "tv": 0.1, "mae": 0.2}]}
    text = diag.report(res)
    assert "quant (no g)" in text and "quant-c [0.9 m, 0.8 M]" in text
