"""The pipelined decode schedule (CQ_PATH_FAST_PIPE: b = 1, up to 8192 visual
tokens and 128 text tokens) on the GPU.

It reads every key tile once and keeps the visual scores on chip until the
value tiles of the same slot use them, while the key tiles of the next
(batch, kv head) unit stream in (QbitAI article on CalibQuant, "Method" parts
2 and 3: post-scaled scores, the calibration map fixed by their min and max,
post-scaled values).  Its outputs must be within 2e-3 of the oracle's.  Its
scores are the one-launch schedule's, but its sums and its text tail are
formed in another order, so the two agree to that tolerance, not bit for bit.
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
PIPE, ONE = cqb.CQ_PATH_FAST_PIPE, cqb.CQ_PATH_FAST_ONE


def _quantize(K, V):
    return cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K), cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)


def _both(K, V, q, kt, vt, calib, out_dtype=None):
    import torch
    n = K.shape[2]
    (kc, ks, km), (vc, vs, vm) = _quantize(K, V)
    outs = []
    for path in (PIPE, ONE):
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


def _close(a, b, tol=REL_TOL):
    err = rel_err(a.float().cpu().numpy(), b.float().cpu().numpy().astype(np.float64))
    assert err <= tol, f"pipelined vs one-launch: {err:.3e}"


@pytest.mark.parametrize("n", [32, 96, 128, 1152, 4224, 8192])
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("T", [0, 64, 128])
def test_tile_counts_groups_tails(n, G, T):
    """Fewer tiles than waves, one to eight tiles per wave, ragged last tile,
    every group size, no tail, one and two tail rounds."""
    K, V, q, kt, vt = draw_inputs(2, 2 * G, 2, n, T, seed=n + 7 * G + T, host=False)
    note(f"decode pipe n={n} G={G} T={T}")
    pipe, one = _both(K, V, q, kt if T else None, vt if T else None, RELATIVE)
    _close(pipe, one)
    _check_oracle(pipe, K, V, q, kt if T else None, vt if T else None, RELATIVE, [(0, 0), (1, 1)])


@pytest.mark.parametrize("B,n", [(96, 1024), (75, 2080), (33, 8192)])
@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE, IDENTITY])
def test_units_walked_per_workgroup(B, n, calib):
    """More (batch, kv head) units than CUs: a workgroup walks two or three in
    turn, the value tiles of one beside the key tiles of the next; with a
    ragged count some workgroups walk one unit fewer."""
    K, V, q, kt, vt = draw_inputs(B, 32, 8, n, 64, seed=17 + B, host=False)
    note(f"decode pipe {B * 8} units n={n} calib={calib}")
    pipe, one = _both(K, V, q, kt, vt, calib)
    _close(pipe, one)
    _check_oracle(pipe, K, V, q, kt, vt, calib, [(0, 0), (B // 3, 7), (B // 2, 0), (B - 1, 7)])


@pytest.mark.parametrize("out_dtype", ["float16", "float32"])
def test_fp32_query_tail_and_output(out_dtype):
    import torch
    K, V, q, kt, vt = draw_inputs(3, 8, 2, 640, 48, dtype="float32", seed=23, host=False)
    note(f"decode pipe fp32 inputs out={out_dtype}")
    pipe, one = _both(K, V, q, kt, vt, RELATIVE, out_dtype=getattr(torch, out_dtype))
    _close(pipe, one)
    _check_oracle(pipe, K, V, q, kt, vt, RELATIVE, [(0, 0), (2, 1)])


def test_shapes_refused():
    """Past 8192 tokens, past 128 tail tokens, a group of 8 or an empty visual
    cache: refused before any launch (the automatic choice takes another
    schedule)."""
    import torch
    for (Hq, n, T) in [(8, 8192 + 128, 0), (8, 256, 129), (16, 256, 0)]:
        K, V, q, kt, vt = draw_inputs(1, Hq, 2, n, T, seed=41, host=False)
        (kc, ks, km), (vc, vs, vm) = _quantize(K, V)
        with pytest.raises(cqb.CQError) as ei:
            cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt if T else None, vt if T else None, n=n, bits=1,
                               sm_scale=SM, path=PIPE)
        assert ei.value.status == 2
    _, _, q, kt, vt = draw_inputs(2, 8, 2, 0, 16, seed=9, host=False)
    z = torch.zeros((2, 2, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(cqb.CQError) as ei:
        cqb.cq_decode_attn(q, None, z, z, None, z, z, kt, vt, n=0, bits=1, sm_scale=SM, path=PIPE)
    assert ei.value.status == 2


def test_long_context_headline():
    """The long-context shape (64 sequences, 32q/8kv, n = 8192, T = 64): 512
    units, two per workgroup on a 256-CU MI355X."""
    K, V, q, kt, vt = draw_inputs(64, 32, 8, 8192, 64, seed=3, host=False)
    note("decode pipe long context")
    pipe, one = _both(K, V, q, kt, vt, RELATIVE)
    _close(pipe, one)
    _check_oracle(pipe, K, V, q, kt, vt, RELATIVE, [(0, 0), (40, 2), (63, 7)])


def test_repeated_calls_are_identical():
    """The schedule keeps no state between calls: three calls give the same bits."""
    import torch
    K, V, q, kt, vt = draw_inputs(40, 32, 8, 3328, 64, seed=5, host=False)
    (kc, ks, km), (vc, vs, vm) = _quantize(K, V)
    note("decode pipe repeated calls")
    outs = [cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=3328, bits=1, sm_scale=SM, calib=RELATIVE,
                               path=PIPE) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
