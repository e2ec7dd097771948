"""The drop-in decode module and its graph-captured multi-layer step (GPU).

CalibQuant is plug-and-play: the visual cache is quantized at prefill and
each decode step attends over the codes and the full-precision text tokens
(CalibQuant abstract; QbitAI article, "Method").  The module must give the
library's own result bit for bit, the oracle's within 2e-3, and a replayed
HIP graph of several layers the eager results bit for bit on every replay.
"""
import numpy as np
import pytest

from helpers import REL_TOL, calib_f32, draw_inputs, note, oracle_unit_decode, rel_err

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")
from extreme_bit_kv_amd.attention import CalibQuantAttention, GraphedDecode, QuantizedVisualKV  # noqa: E402

SM = 1.0 / np.sqrt(128.0)
RELATIVE = (0.9, 0.0, 0.8, 0.0)


def test_module_matches_library_and_oracle():
    import torch
    B, Hq, Hkv, n, T = 2, 8, 2, 512, 16
    K, V, q, kt, vt = draw_inputs(B, Hq, Hkv, n, T, seed=31)
    note("attention module B=2 8q/2kv n=512 T=16")
    cache = QuantizedVisualKV(K, V, bits=1)
    attn = CalibQuantAttention(SM, RELATIVE)
    got = attn(q, cache, kt, vt)
    direct = cqb.cq_decode_attn(q, *cache.k, *cache.v, kt, vt, n=n, bits=1, sm_scale=SM, calib=RELATIVE)
    torch.cuda.synchronize()
    assert torch.equal(got, direct)
    G = Hq // Hkv
    worst = 0.0
    for b in range(B):
        for h in range(Hkv):
            ref = oracle_unit_decode(q[b, h * G:(h + 1) * G].cpu().numpy(), K[b, h].cpu().numpy(),
                                     V[b, h].cpu().numpy(), kt[b, h].cpu().numpy(), vt[b, h].cpu().numpy(),
                                     1, SM, calib_f32(RELATIVE))
            worst = max(worst, rel_err(got[b, h * G:(h + 1) * G].float().cpu().numpy(), ref))
    assert worst <= REL_TOL, f"relative error {worst:.3e}"
    assert cache.nbytes == (2 * B * Hkv * n * 128 // 8) + 4 * B * Hkv * 128 * 4


@pytest.mark.parametrize("B,Hkv", [(2, 2), (16, 8)])     # split schedule (4 units), one launch (128 units)
def test_graphed_decode_replays_match_eager(B, Hkv):
    import torch
    layers, Hq, n, T = 4, 4 * Hkv, 1024, 64
    note(f"graphed decode {layers} layers B={B} {Hq}q/{Hkv}kv n={n} T={T}")
    attn = CalibQuantAttention(SM, RELATIVE)
    stack, qs = [], []
    for layer in range(layers):
        K, V, q, kt, vt = draw_inputs(B, Hq, Hkv, n, T, seed=40 + layer, host=False)
        stack.append((attn, QuantizedVisualKV(K, V, bits=1), kt, vt))
        qs.append(q)
    g = GraphedDecode(stack, qs)
    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        new_q = [torch.randn(q.shape, generator=gen, device="cuda").to(q.dtype) for q in qs]
        eager = [a(q, c, kt, vt).clone() for (a, c, kt, vt), q in zip(stack, new_q)]
        torch.cuda.synchronize()
        outs = g.step(new_q)
        torch.cuda.synchronize()
        for layer, (e, o) in enumerate(zip(eager, outs)):
            assert torch.equal(e, o), f"replay {rep}, layer {layer} differs from the eager call"
        # unrelated eager work between replays
        x = torch.randn(256, 256, device="cuda")
        (x @ x).sum().item()
