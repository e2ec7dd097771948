"""The all-in-flight decode schedule (CQ_PATH_FAST_WIDE) on the GPU.

Each (batch, kv head) unit's workgroup requests every code tile it will use at
once and keeps its visual scores in registers between the key pass and the
value pass (QbitAI article on CalibQuant, "Method" parts 2 and 3: post-scaled
scores, the calibration map fixed by their min and max, post-scaled values).
It computes what the one-launch schedule computes, so its outputs must equal
CQ_PATH_FAST_ONE's bit for bit, and the oracle's within 2e-3.  Shapes cross
the boundary between two and four tiles per wave (n = 2048 / 2080), the
largest length it takes (n = 4096) and one past it, fewer tiles than waves
and a ragged last tile.
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
WIDE, ONE = cqb.CQ_PATH_FAST_WIDE, cqb.CQ_PATH_FAST_ONE


def _both(K, V, q, kt, vt, calib, out_dtype=None):
    import torch
    n = K.shape[2]
    kc, ks, km = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
    outs = []
    for path in (WIDE, ONE):
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


@pytest.mark.parametrize("n", [32, 96, 128, 1056, 2048, 2080, 3328, 4096])
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("T", [0, 64, 200])
def test_equals_one_launch(n, G, T):
    import torch
    K, V, q, kt, vt = draw_inputs(2, 2 * G, 2, n, T, seed=n + 7 * G + T + 5, host=False)
    note(f"decode wide n={n} G={G} T={T}")
    wide, one = _both(K, V, q, kt if T else None, vt if T else None, RELATIVE)
    assert torch.equal(wide, one), "the all-in-flight schedule differs from the one-launch schedule"
    _check_oracle(wide, K, V, q, kt if T else None, vt if T else None, RELATIVE, [(0, 0), (1, 1)])


@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE, IDENTITY])
def test_bit_sweep_shape(calib):
    """32 sequences, 32q/8kv, n = 3328, T = 64: 256 units, one per CU on a
    256-CU MI355X (the shape this schedule is chosen for)."""
    import torch
    K, V, q, kt, vt = draw_inputs(32, 32, 8, 3328, 64, seed=31, host=False)
    note(f"decode wide 256 units calib={calib}")
    wide, one = _both(K, V, q, kt, vt, calib)
    assert torch.equal(wide, one)
    _check_oracle(wide, K, V, q, kt, vt, calib, [(0, 0), (13, 5), (31, 7)])


def test_more_units_than_cus():
    """The schedule is correct at any unit count (it is only slow once units
    queue for CUs); AUTO does not choose it there."""
    import torch
    K, V, q, kt, vt = draw_inputs(80, 32, 8, 512, 16, seed=32, host=False)   # 640 units
    note("decode wide 640 units")
    wide, one = _both(K, V, q, kt, vt, RELATIVE)
    assert torch.equal(wide, one)
    _check_oracle(wide, K, V, q, kt, vt, RELATIVE, [(0, 0), (79, 7)])


@pytest.mark.parametrize("out_dtype", ["float16", "float32"])
def test_fp32_query_tail_and_output(out_dtype):
    import torch
    K, V, q, kt, vt = draw_inputs(3, 8, 2, 640, 48, dtype="float32", seed=33, host=False)
    note(f"decode wide fp32 inputs out={out_dtype}")
    wide, one = _both(K, V, q, kt, vt, RELATIVE, out_dtype=getattr(torch, out_dtype))
    assert torch.equal(wide, one)
    _check_oracle(wide, K, V, q, kt, vt, RELATIVE, [(0, 0), (2, 1)])


def test_tail_only():
    """n = 0: the text tail alone."""
    import torch
    _, _, q, kt, vt = draw_inputs(2, 8, 2, 0, 16, seed=34, host=False)
    z = torch.zeros((2, 2, 128), dtype=torch.float32, device="cuda")
    note("decode wide n=0")
    outs = [cqb.cq_decode_attn(q, None, z, z, None, z, z, kt, vt, n=0, bits=1, sm_scale=SM, calib=RELATIVE, path=p)
            for p in (WIDE, ONE)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_refused_past_its_length():
    """n = 4128 needs a fifth tile per wave: refused before any launch."""
    K, V, q, _, _ = draw_inputs(1, 4, 1, 4128, 0, seed=35, host=False)
    kc, ks, km = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
    with pytest.raises(cqb.CQError) as ei:
        cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, None, None, n=4128, bits=1, sm_scale=SM, path=WIDE)
    assert ei.value.status == 2
