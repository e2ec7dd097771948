"""Decode with a text tail longer than the fused pass holds (T > 256) on the
one-launch schedules, against the oracle.

Only the visual cache is quantized (QbitAI article on CalibQuant, abstract);
the text tail is attended in full precision beside the post-scaled visual
products ("Method" part 2), and the softmax runs over both.  A long tail is
taken in chunks of 256 tokens with a running reference, so the cases below
cover one token past a chunk, whole chunks, many chunks, a tail token that
dominates every visual score and a tail far below the visual scores.
Outputs must be within 2e-3 of the oracle (inf-norm per head vector).
"""
import numpy as np
import pytest

from helpers import REL_TOL, calib_f32, draw_inputs, note, oracle_unit_decode, rel_err

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")

SM = 1.0 / np.sqrt(128.0)
RELATIVE = (0.9, 0.0, 0.8, 0.0)
PATHS = [cqb.CQ_PATH_AUTO, cqb.CQ_PATH_FAST, cqb.CQ_PATH_FAST_ONE]


def _check(K, V, q, kt, vt, bits, calib, path, out_dtype=None):
    import torch
    B, Hkv, n, _ = K.shape
    G = q.shape[1] // Hkv
    kc, ks, km = cqb.cq_quantize_kv(K, bits, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V, bits, cqb.CQ_LAYOUT_V)
    out = cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=bits, sm_scale=SM, calib=calib,
                             path=path, out_dtype=out_dtype or torch.float32)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.all(np.isfinite(got))
    for b in range(B):
        for h in range(Hkv):
            ref = oracle_unit_decode(q[b, h * G:(h + 1) * G].cpu().numpy(), K[b, h].cpu().numpy(),
                                     V[b, h].cpu().numpy(), kt[b, h].cpu().numpy(), vt[b, h].cpu().numpy(),
                                     bits, SM, calib_f32(calib))
            err = rel_err(got[b, h * G:(h + 1) * G], ref)
            assert err <= REL_TOL, f"unit ({b}, {h}): relative error {err:.3e}"


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T", [257, 512, 513, 1024, 4096])
def test_long_tail_b1(T, path):
    K, V, q, kt, vt = draw_inputs(2, 8, 2, 1056, T, seed=T + 1)
    note(f"long tail b=1 T={T} path={path}")
    _check(K, V, q, kt, vt, 1, RELATIVE, path)


@pytest.mark.parametrize("G", [1, 2])
@pytest.mark.parametrize("calib", [None, RELATIVE])
def test_long_tail_groups_calib(G, calib):
    K, V, q, kt, vt = draw_inputs(1, 2 * G, 2, 2080, 1000, seed=7 + G)
    note(f"long tail G={G} calib={calib}")
    _check(K, V, q, kt, vt, 1, calib, cqb.CQ_PATH_FAST_ONE)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("T", [300, 1024])
def test_long_tail_multibit(bits, T):
    K, V, q, kt, vt = draw_inputs(1, 8, 2, 1024, T, seed=bits * 10 + T)
    note(f"long tail bits={bits} T={T}")
    _check(K, V, q, kt, vt, bits, None, cqb.CQ_PATH_AUTO)


def test_long_tail_float32():
    K, V, q, kt, vt = draw_inputs(1, 8, 2, 1024, 700, dtype="float32", seed=5)
    note("long tail float32 T=700")
    _check(K, V, q, kt, vt, 1, RELATIVE, cqb.CQ_PATH_FAST_ONE)


@pytest.mark.parametrize("scale", [40.0, -40.0])
def test_long_tail_far_from_visual(scale):
    """One late tail token far above every visual score (scale 40), or the
    whole tail far below them (-40): the references of the two parts differ
    by far more than a float exponent spans."""
    import torch
    K, V, q, kt, vt = draw_inputs(1, 4, 1, 1056, 1500, seed=11)
    qs = q[0].double().cpu()
    u = qs.sum(0) / qs.sum(0).norm()
    if scale > 0:
        kt[0, 0, 1400] = (u * scale / SM / float(max(1e-3, (qs @ u).min()))).half().to(kt.device)
    else:
        kt[0, 0] = (kt[0, 0].double().cpu() * 0.0 + u * scale / SM / float(max(1e-3, (qs @ u).min()))).half() \
            .to(kt.device)
    note(f"long tail far from visual scale={scale}")
    _check(K, V, q, kt, vt, 1, None, cqb.CQ_PATH_FAST_ONE)
