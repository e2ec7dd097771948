"""Decode between appends: a visual cache that grows frame by frame, decoded
in place after every frame.

The pages motivate CalibQuant with visual tokens that pile up in the cache
(QbitAI article on CalibQuant, "Motivation"); the range of each channel is
taken over all of one head's visual tokens ("Method" part 1), so a new frame
can widen it and change the earlier codes.  The chunked quantizer keeps the
codes of the segment so far in buffers laid out for the whole segment
(n_cap tokens); after each frame the decode attends over the first n of
them (cq_opts.n_cap).  Three frames of 1024, 1024 and 1280 tokens are
appended; after each one, every decode path must give the oracle's output
on the first n tokens within 2e-3, and exactly what the same path gives on
a compact copy of those n tokens quantized in one call.
"""
import numpy as np
import pytest

from helpers import REL_TOL, calib_f32, note, oracle_unit_decode, rel_err
from workloads import ROLE_K, ROLE_KTAIL, ROLE_V, ROLE_VTAIL, kv_torch, q_torch

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")
from extreme_bit_kv_amd.prefill import ChunkedVisualQuantizer  # noqa: E402

SM = 1.0 / np.sqrt(128.0)
RELATIVE = (0.9, 0.0, 0.8, 0.0)
FRAMES = (1024, 1024, 1280)
P = cqb
B1_PATHS = [P.CQ_PATH_GENERIC, P.CQ_PATH_AUTO, P.CQ_PATH_FAST_ONE, P.CQ_PATH_FAST_LDS, P.CQ_PATH_FAST_PIPE,
            P.CQ_PATH_FAST_SPLIT, P.CQ_PATH_FAST_WIDE]
BN_PATHS = [P.CQ_PATH_GENERIC, P.CQ_PATH_AUTO, P.CQ_PATH_FAST_ONE]


@pytest.mark.parametrize("bits,calib", [(1, RELATIVE), (1, None), (2, None), (8, RELATIVE)])
def test_three_frame_append(bits, calib):
    import torch
    B, Hkv, G, T, seed = 2, 2, 4, 16, 61
    cap = sum(FRAMES)
    K = kv_torch(seed, 0, ROLE_K, B, Hkv, cap, 128, "float16", "cuda")
    V = kv_torch(seed, 0, ROLE_V, B, Hkv, cap, 128, "float16", "cuda")
    # later frames drift, so that they widen some channels' ranges
    for f, (a, m) in enumerate(zip(np.cumsum((0,) + FRAMES[:-1]), FRAMES)):
        K[:, :, a:a + m] *= 1.0 + 0.25 * f
        V[:, :, a:a + m] += 0.5 * f
    kt = kv_torch(seed, 0, ROLE_KTAIL, B, Hkv, T, 128, "float16", "cuda")
    vt = kv_torch(seed, 0, ROLE_VTAIL, B, Hkv, T, 128, "float16", "cuda")
    Kh, Vh, kth, vth = (x.cpu().numpy() for x in (K, V, kt, vt))
    cz = ChunkedVisualQuantizer(K, V, cap, bits=bits, eager=True)
    paths = B1_PATHS if bits == 1 else BN_PATHS
    n = 0
    for f, m in enumerate(FRAMES):
        cz.append(m)
        n += m
        cur = cz.current()
        assert cur.n == n and cur.n_cap == cap
        q = q_torch(seed + f, 0, B, Hkv * G, 128, "float16", "cuda")
        qh = q.cpu().numpy()
        ref = np.zeros(qh.shape)
        for b in range(B):
            for h in range(Hkv):
                ref[b, h * G:(h + 1) * G] = oracle_unit_decode(qh[b, h * G:(h + 1) * G], Kh[b, h, :n], Vh[b, h, :n],
                                                               kth[b, h], vth[b, h], bits, SM, calib_f32(calib))
        kc, ks, km = cqb.cq_quantize_kv(K[:, :, :n].contiguous(), bits, cqb.CQ_LAYOUT_K)
        vc, vs, vm = cqb.cq_quantize_kv(V[:, :, :n].contiguous(), bits, cqb.CQ_LAYOUT_V)
        for path in paths:
            note(f"append bits={bits} calib={calib} frame={f} n={n} path={path}")
            got = cqb.cq_decode_attn(q, *cur.k, *cur.v, kt, vt, n=n, bits=bits, sm_scale=SM, calib=calib, path=path,
                                     n_cap=cap, out_dtype=torch.float32)
            compact = cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=bits, sm_scale=SM,
                                         calib=calib, path=path, out_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(got, compact), f"path {path}: the in-place decode differs from the compact one"
            err = rel_err(got.cpu().numpy(), ref)
            assert err <= REL_TOL, f"path {path}: relative error {err:.3e}"
    assert cz.t == cap


def test_module_decodes_the_segment_so_far():
    """CalibQuantAttention over QuantizedVisualKV.from_codes(..., n_cap)."""
    import torch
    from extreme_bit_kv_amd.attention import CalibQuantAttention
    B, Hkv, G, cap, seed = 1, 2, 4, 2048, 62
    K = kv_torch(seed, 0, ROLE_K, B, Hkv, cap, 128, "float16", "cuda")
    V = kv_torch(seed, 0, ROLE_V, B, Hkv, cap, 128, "float16", "cuda")
    cz = ChunkedVisualQuantizer(K, V, cap, eager=True)
    cz.append(1024)
    q = q_torch(seed, 0, B, Hkv * G, 128, "float16", "cuda")
    attn = CalibQuantAttention(SM, RELATIVE)
    note("append module n=1024 of 2048")
    got = attn(q, cz.current())
    kc, ks, km = cqb.cq_quantize_kv(K[:, :, :1024].contiguous(), 1, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V[:, :, :1024].contiguous(), 1, cqb.CQ_LAYOUT_V)
    want = cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, None, None, n=1024, bits=1, sm_scale=SM, calib=RELATIVE)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
