"""GPU calibration map and fp16 baseline vs the oracle."""
import numpy as np
import pytest

import oracle
from helpers import REL_TOL, calib_f32, note, rel_err
from workloads import ROLE_K, ROLE_V, kv_numpy, q_numpy

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")


@pytest.mark.parametrize("calib", [(0.9, 0.0, 0.8, 0.0), (0.0, -4.0, 0.0, 4.0), (0.5, 1.0, -1.0, 2.0),
                                   (1.0, 0.0, 1.0, 0.0)])
@pytest.mark.parametrize("R,n", [(1, 1), (3, 257), (64, 3328)])
def test_calibrate_matches_oracle(calib, R, n):
    import torch
    rng = np.random.default_rng(R + n)
    s = (rng.standard_normal((R, n)) * 3).astype(np.float32)
    s[:, :1] = 1.25 if n == 1 else s[:, :1]
    sd = torch.from_numpy(s).cuda()
    mm = torch.empty((R, 2), dtype=torch.float32, device="cuda")
    note(f"calibrate R={R} n={n} calib={calib}")
    out = cqb.cq_calibrate(sd, calib, row_minmax=mm)
    torch.cuda.synchronize()
    ref, m, M = oracle.calibrate_rows(s.astype(np.float64), calib_f32(calib))
    got = out.cpu().numpy()
    # computed in float64 and rounded once: within one float32 ulp of the oracle
    assert np.all(np.abs(got - ref) <= np.spacing(np.abs(ref).astype(np.float32)) + 1e-30)
    assert np.array_equal(mm.cpu().numpy(), np.stack([m, M], -1).astype(np.float32))


def test_calibrate_in_place_and_disabled():
    import torch
    s = torch.randn((4, 100), device="cuda")
    ref = s.clone()
    note("calibrate in place")
    cqb.cq_calibrate(s, None, out=s)           # disabled: copy
    torch.cuda.synchronize()
    assert torch.equal(s, ref)
    cqb.cq_calibrate(s, (0.9, 0.0, 0.8, 0.0), out=s)
    torch.cuda.synchronize()
    exp, _, _ = oracle.calibrate_rows(ref.cpu().numpy().astype(np.float64), calib_f32((0.9, 0.0, 0.8, 0.0)))
    assert np.allclose(s.cpu().numpy(), exp, rtol=2e-7, atol=1e-7)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 4, 1, 1), (2, 8, 2, 777), (3, 32, 8, 3392), (1, 8, 8, 2048),
                                         (2, 6, 2, 65), (1, 16, 2, 130), (1, 7, 1, 63), (1, 10, 2, 5000),
                                         (2, 24, 8, 8256)])
def test_fp16_baseline_matches_textbook_attention(B, Hq, Hkv, N):
    import torch
    K = kv_numpy(40 + N, 0, ROLE_K, B, Hkv, N, 128)
    V = kv_numpy(40 + N, 0, ROLE_V, B, Hkv, N, 128)
    q = q_numpy(40 + N, 0, B, Hq, 128)
    sm = 1 / np.sqrt(128)
    note(f"fp16 baseline B={B} Hq={Hq} Hkv={Hkv} N={N}")
    out = cqb.cq_decode_attn_fp16(torch.from_numpy(q).cuda(), torch.from_numpy(K).cuda(),
                                  torch.from_numpy(V).cuda(), sm)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            ref = oracle.attend_dense(q[b, h * G:(h + 1) * G], K[b, h], V[b, h], sm)
            assert rel_err(got[b, h * G:(h + 1) * G], ref) <= REL_TOL
