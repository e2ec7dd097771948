"""GPU pre-softmax scores vs the oracle: cq_visual_scores (post-scaled codes,
QbitAI article on CalibQuant, "Method" part 2), calibrated by cq_calibrate
(part 3), and the exact cq_scores_fp16 over an unquantized cache.  Scores are
float32 with float32 accumulation: within 1e-5 of the row's largest |score|."""
import numpy as np
import pytest

import oracle
from helpers import calib_f32, draw_inputs, note

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")

SM = 1.0 / np.sqrt(128.0)
TOL = 1e-5


def _close(got, ref):
    scale = np.maximum(np.abs(ref).max(axis=-1, keepdims=True), 1e-30)
    err = float((np.abs(got - ref) / scale).max())
    assert err <= TOL, f"max error {err:.3e} of the row scale"


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("G,n", [(1, 1), (4, 100), (4, 3328), (8, 257)])
@pytest.mark.parametrize("qdt", ["float16", "float32"])
def test_visual_scores(bits, G, n, qdt):
    import torch
    Hkv = 2
    K, _, q, _, _ = draw_inputs(2, G * Hkv, Hkv, n, 0, seed=bits * 31 + n + G)
    if qdt == "float32":
        q = q.float()
    kc, ks, km = cqb.cq_quantize_kv(K, bits, cqb.CQ_LAYOUT_K)
    note(f"visual scores bits={bits} G={G} n={n} q={qdt}")
    got = cqb.cq_visual_scores(q, kc, ks, km, n=n, bits=bits, sm_scale=SM)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    _, ks_o, km_o, codes = oracle.quantize(K.cpu().numpy(), bits, "K")
    qn = q.float().cpu().numpy()
    for b in range(2):
        for h in range(Hkv):
            ref = oracle.visual_scores(qn[b, h * G:(h + 1) * G], codes[b, h], ks_o[b, h], km_o[b, h], SM)
            _close(got[b, h * G:(h + 1) * G], ref)


@pytest.mark.parametrize("calib", [(0.9, 0.0, 0.8, 0.0), (0.0, -4.0, 0.0, 4.0)])
def test_calibrated_visual_scores(calib):
    """The calibrated scores the decode softmax sees: g of each query-head row."""
    import torch
    K, _, q, _, _ = draw_inputs(2, 8, 2, 800, 0, seed=99)
    kc, ks, km = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
    note(f"calibrated visual scores calib={calib}")
    s = cqb.cq_visual_scores(q, kc, ks, km, n=800, bits=1, sm_scale=SM)
    got = cqb.cq_calibrate(s.view(-1, 800), calib).view(2, 8, 800)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    _, ks_o, km_o, codes = oracle.quantize(K.cpu().numpy(), 1, "K")
    qn = q.float().cpu().numpy()
    for b in range(2):
        for h in range(2):
            raw = oracle.visual_scores(qn[b, 4 * h:4 * h + 4], codes[b, h], ks_o[b, h], km_o[b, h], SM)
            ref, _, _ = oracle.calibrate_rows(raw, calib_f32(calib))
            _close(got[b, 4 * h:4 * h + 4], ref)


@pytest.mark.parametrize("G,N", [(1, 1), (4, 63), (4, 3392), (3, 200), (8, 1000)])
def test_scores_fp16(G, N):
    import torch
    Hkv = 2
    K, _, q, _, _ = draw_inputs(2, G * Hkv, Hkv, N, 0, seed=N + 7 * G)
    note(f"fp16 scores G={G} N={N}")
    got = cqb.cq_scores_fp16(q, K, SM)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    Kn, qn = K.cpu().numpy(), q.cpu().numpy()
    for b in range(2):
        for h in range(Hkv):
            _close(got[b, h * G:(h + 1) * G], oracle.dense_scores(qn[b, h * G:(h + 1) * G], Kn[b, h], SM))


def test_score_distribution_diagnostic():
    """The diagnostic's numbers against the oracle's scores; the identity map changes nothing."""
    from extreme_bit_kv_amd import diagnostics as diag
    K, _, q, _, _ = draw_inputs(1, 8, 2, 512, 0, seed=5)
    note("score-distribution diagnostic")
    res = diag.score_distribution(K, q, sm_scale=SM, calibs=[(1.0, 0.0, 1.0, 0.0), (0.9, 0.0, 0.8, 0.0)])
    quant, ident, rel = res["settings"]
    assert ident["kl_mean"] == pytest.approx(quant["kl_mean"], rel=1e-6)
    assert min(quant["kl_mean"], rel["kl_mean"]) >= 0.0
    assert sum(res["exact_hist"]) == pytest.approx(1.0)
    # the same KL from the oracle's exact and quantized scores
    _, ks_o, km_o, codes = oracle.quantize(K.cpu().numpy(), 1, "K")
    qn, Kn = q.float().cpu().numpy(), K.cpu().numpy()
    kls = []
    for h in range(2):
        ex = oracle.dense_scores(qn[0, 4 * h:4 * h + 4], Kn[0, h], SM)
        qs = oracle.visual_scores(qn[0, 4 * h:4 * h + 4], codes[0, h], ks_o[0, h], km_o[0, h], SM)
        kls.append(diag.kl_rows(ex, qs))
    assert quant["kl_mean"] == pytest.approx(float(np.mean(np.concatenate(kls))), rel=1e-3)
