"""The LDS-score decode schedule (CQ_PATH_FAST_LDS) on the GPU.

It computes what the one-launch schedule computes, with the visual scores
kept in LDS between the key and the value pass instead of recomputed from a
second read of the keys (QbitAI article on CalibQuant, "Method" parts 2 and 3:
post-scaled scores, the calibration map fixed by their min and max, post-scaled
values).  Its outputs must equal CQ_PATH_FAST_ONE's bit for bit, and the
oracle's within 2e-3; a workgroup walks several (batch, kv head) units when
there are more units than CUs.
"""
import numpy as np
import pytest

from helpers import REL_TOL, calib_f32, draw_inputs, note, oracle_unit_decode, rel_err

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")

SM = 1.0 / np.sqrt(128.0)
RELATIVE = (0.9, 0.0, 0.8, 0.0)
ABSOLUTE = (0.0, -4.0, 0.0, 4.0)
IDENTITY = (1.0, 0.0, 1.0, 0.0)
LDS, ONE = cqb.CQ_PATH_FAST_LDS, cqb.CQ_PATH_FAST_ONE


def _both(K, V, q, kt, vt, calib, out_dtype=None):
    import torch
    n = K.shape[2]
    kc, ks, km = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
    outs = []
    for path in (LDS, ONE):
        outs.append(cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=1, sm_scale=SM, calib=calib,
                                       path=path, out_dtype=out_dtype))
    torch.cuda.synchronize()
    return outs


def _check_oracle(got, K, V, q, kt, vt, calib, units):
    G = q.shape[1] // K.shape[1]
    g = got.float().cpu().numpy()
    worst = 0.0
    for b, h in units:
        ref = oracle_unit_decode(q[b, h * G:(h + 1) * G].cpu().numpy(), K[b, h].cpu().numpy(),
                                 V[b, h].cpu().numpy(), None if kt is None else kt[b, h].cpu().numpy(),
                                 None if vt is None else vt[b, h].cpu().numpy(), 1, SM, calib_f32(calib))
        worst = max(worst, rel_err(g[b, h * G:(h + 1) * G], ref))
    assert worst <= REL_TOL, f"relative error {worst:.3e}"


@pytest.mark.parametrize("n", [32, 96, 128, 1152, 4224, 8192])
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("T", [0, 64, 200])
def test_equals_one_launch(n, G, T):
    """Fewer tiles than waves, one and several tiles per wave, ragged last tile."""
    import torch
    K, V, q, kt, vt = draw_inputs(2, 2 * G, 2, n, T, seed=n + 7 * G + T, host=False)
    note(f"decode lds n={n} G={G} T={T}")
    lds, one = _both(K, V, q, kt if T else None, vt if T else None, RELATIVE)
    assert torch.equal(lds, one), "the LDS-score schedule differs from the one-launch schedule"
    _check_oracle(lds, K, V, q, kt if T else None, vt if T else None, RELATIVE, [(0, 0), (1, 1)])


@pytest.mark.parametrize("G,n", [(4, 8192), (2, 16384), (1, 32768)])
def test_largest_segment_per_group(G, n):
    """G x ceil(n / 128) = 256: the whole 128 KB of scores in use."""
    import torch
    K, V, q, kt, vt = draw_inputs(1, 2 * G, 2, n, 64, seed=40 + G, host=False)
    note(f"decode lds capacity G={G} n={n}")
    lds, one = _both(K, V, q, kt, vt, RELATIVE)
    assert torch.equal(lds, one)
    _check_oracle(lds, K, V, q, kt, vt, RELATIVE, [(0, 0), (0, 1)])
    # one tile more than fits: refused before any launch
    K2, V2, q2, kt2, vt2 = draw_inputs(1, 2 * G, 2, n + 128, 0, seed=41, host=False)
    kc, ks, km = cqb.cq_quantize_kv(K2, 1, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V2, 1, cqb.CQ_LAYOUT_V)
    with pytest.raises(cqb.CQError) as ei:
        cqb.cq_decode_attn(q2, kc, ks, km, vc, vs, vm, None, None, n=n + 128, bits=1, sm_scale=SM, path=LDS)
    assert ei.value.status == 2


@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE, IDENTITY])
def test_units_walked_per_workgroup(calib):
    """More (batch, kv head) units than CUs: each workgroup takes several in
    turn (and requests the next one's inputs during the current one)."""
    import torch
    K, V, q, kt, vt = draw_inputs(96, 32, 8, 1024, 64, seed=17, host=False)   # 768 units
    note(f"decode lds 768 units calib={calib}")
    lds, one = _both(K, V, q, kt, vt, calib)
    assert torch.equal(lds, one)
    _check_oracle(lds, K, V, q, kt, vt, calib, [(0, 0), (31, 7), (32, 0), (95, 7)])


@pytest.mark.parametrize("out_dtype", ["float16", "float32"])
def test_fp32_query_tail_and_output(out_dtype):
    import torch
    K, V, q, kt, vt = draw_inputs(3, 8, 2, 640, 48, dtype="float32", seed=23, host=False)
    note(f"decode lds fp32 inputs out={out_dtype}")
    lds, one = _both(K, V, q, kt, vt, RELATIVE, out_dtype=getattr(torch, out_dtype))
    assert torch.equal(lds, one)
    _check_oracle(lds, K, V, q, kt, vt, RELATIVE, [(0, 0), (2, 1)])


def test_tail_only():
    """n = 0: the text tail alone."""
    import torch
    _, _, q, kt, vt = draw_inputs(2, 8, 2, 0, 16, seed=9, host=False)
    z = torch.zeros((2, 2, 128), dtype=torch.float32, device="cuda")
    note("decode lds n=0")
    outs = [cqb.cq_decode_attn(q, None, z, z, None, z, z, kt, vt, n=0, bits=1, sm_scale=SM, calib=RELATIVE, path=p)
            for p in (LDS, ONE)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_long_context_headline():
    """The long-context shape (64 sequences, 32q/8kv, n = 8192, T = 64): 512
    units on the CUs, two per workgroup on a 256-CU MI355X."""
    import torch
    K, V, q, kt, vt = draw_inputs(64, 32, 8, 8192, 64, seed=3, host=False)
    note("decode lds long context")
    lds, one = _both(K, V, q, kt, vt, RELATIVE)
    assert torch.equal(lds, one)
    _check_oracle(lds, K, V, q, kt, vt, RELATIVE, [(0, 0), (40, 2), (63, 7)])
