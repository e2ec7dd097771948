"""cq_decode_attn_noalloc on the GPU: the decode with the library's fixed
per-device scratch instead of a caller's workspace.

Its outputs must equal cq_decode_attn's (same schedule, same opts, a workspace
from the caller) bit for bit, on two calls in a row, the second one smaller,
so that the scratch left by the first call cannot leak into the second.  The
small case of each schedule is also checked against the oracle to the decode
tolerance (QbitAI article on CalibQuant, "Method" parts 2 and 3).
"""
import gc

import numpy as np
import pytest

from helpers import REL_TOL, calib_f32, draw_inputs, note, oracle_unit_decode, rel_err

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")

SM = 1.0 / np.sqrt(128.0)
RELATIVE = (0.9, 0.0, 0.8, 0.0)


def _inputs(B, Hq, Hkv, n, T, bits, seed):
    import torch
    K, V, q, kt, vt = draw_inputs(B, Hq, Hkv, n, T, seed=seed, host=False)
    kc, ks, km = cqb.cq_quantize_kv(K, bits, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V, bits, cqb.CQ_LAYOUT_V)
    torch.cuda.synchronize()
    return (K, V, q, kt, vt), (q, kc, ks, km, vc, vs, vm, kt, vt)


def _both(args, n, bits, path, calib, splits=0):
    """(with a workspace, without) outputs of one decode, float32."""
    import torch
    q = args[0]
    ref = cqb.cq_decode_attn(*args, n=n, bits=bits, sm_scale=SM, calib=calib, path=path, splits=splits,
                             out_dtype=torch.float32)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    # the collector could free an earlier test's tensors in the middle of the
    # call and make the count drop: collect first, and keep it off meanwhile
    gc.collect()
    gc.disable()
    try:
        before = torch.cuda.memory_allocated()
        cqb.cq_decode_attn_noalloc(*args, n=n, bits=bits, sm_scale=SM, calib=calib, path=path, splits=splits,
                                   out=out)
        torch.cuda.synchronize()
        after = torch.cuda.memory_allocated()
    finally:
        gc.enable()
    assert after == before
    return ref, out


def _oracle_check(raw, got, bits, calib, B, Hq, Hkv):
    K, V, q, kt, vt = (None if t is None else t.cpu().numpy() for t in raw)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            ref = oracle_unit_decode(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], None if kt is None else kt[b, h],
                                     None if vt is None else vt[b, h], bits, SM, calib_f32(calib))
            err = rel_err(got[b, h * G:(h + 1) * G], ref)
            assert err <= REL_TOL, f"unit ({b}, {h}): relative error {err:.3e}"


# (path, bits, splits, first shape, second (smaller) shape); a shape is (B, Hq, Hkv, n, T)
CASES = [
    ("split", cqb.CQ_PATH_FAST_SPLIT, 1, 0, (8, 32, 8, 8192, 64), (2, 16, 4, 2080, 16)),
    ("split_chunks", cqb.CQ_PATH_FAST_SPLIT, 1, 8, (4, 32, 8, 4096, 0), (1, 8, 8, 1024, 8)),
    ("auto_small_batch", cqb.CQ_PATH_AUTO, 1, 0, (2, 32, 8, 16384, 32), (1, 32, 8, 12288, 0)),   # split schedule
    ("generic_b2", cqb.CQ_PATH_GENERIC, 2, 0, (2, 32, 8, 4096, 48), (1, 8, 2, 1000, 5)),
    ("generic_b1", cqb.CQ_PATH_GENERIC, 1, 0, (2, 16, 8, 2048, 16), (1, 4, 4, 96, 0)),
    ("one_b4", cqb.CQ_PATH_FAST_ONE, 4, 0, (2, 32, 8, 2048, 16), (1, 16, 8, 512, 0)),
]


@pytest.mark.parametrize("label,path,bits,splits,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_decode(label, path, bits, splits, first, second):
    for step, shape in enumerate((first, second)):
        B, Hq, Hkv, n, T = shape
        note(f"noalloc {label} call {step} B={B} Hq={Hq} Hkv={Hkv} n={n} T={T} bits={bits}")
        raw, args = _inputs(B, Hq, Hkv, n, T, bits, seed=11 + step)
        ref, got = _both(args, n, bits, path, RELATIVE, splits)
        assert bool(got.isfinite().all())
        assert bool((got == ref).all()), f"call {step}: max diff {(got - ref).abs().max().item():.3e}"
        if step == 1:
            _oracle_check(raw, got.cpu().numpy(), bits, RELATIVE, B, Hq, Hkv)


def test_noalloc_rejects_what_exceeds_the_scratch():
    """The generic schedule's score buffer at 64 x 32 heads x 8192 tokens is
    64 MiB: more than the fixed scratch, so the call is refused up front."""
    import torch
    B, Hq, Hkv, n, T = 64, 32, 8, 8192, 0
    raw, args = _inputs(B, Hq, Hkv, n, T, 1, seed=3)
    out = torch.zeros((B, Hq, 128), dtype=torch.float16, device="cuda")
    note("noalloc oversize generic")
    with pytest.raises(cqb.CQError) as ei:
        cqb.cq_decode_attn_noalloc(*args, n=n, bits=1, sm_scale=SM, path=cqb.CQ_PATH_GENERIC, out=out)
    assert ei.value.status == 3                    # CQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 0).all())                  # nothing was enqueued
