"""GPU decode attention vs the oracle (QbitAI article on CalibQuant, "Method"
parts 2 and 3): relative error <= 2e-3 per head vector (inf-norm)."""
import numpy as np
import pytest

import oracle
from helpers import REL_TOL, calib_f32, draw_inputs, note, oracle_unit_decode, rel_err

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")

SM = 1.0 / np.sqrt(128.0)
RELATIVE = (0.9, 0.0, 0.8, 0.0)
ABSOLUTE = (0.0, -4.0, 0.0, 4.0)
IDENTITY = (1.0, 0.0, 1.0, 0.0)
PATHS = [cqb.CQ_PATH_GENERIC, cqb.CQ_PATH_AUTO, cqb.CQ_PATH_FAST, cqb.CQ_PATH_FAST_ONE, cqb.CQ_PATH_FAST_SPLIT]
FAST_PATHS = (cqb.CQ_PATH_FAST, cqb.CQ_PATH_FAST_ONE, cqb.CQ_PATH_FAST_SPLIT)


def fast_ok(q, K, kt, bits, path=cqb.CQ_PATH_FAST):
    """Shapes the matrix-core decode schedules take (else CQ_ERR_UNSUPPORTED)."""
    n, G = K.shape[2], q.shape[1] // K.shape[1]
    T = 0 if kt is None else kt.shape[2]
    common = G in (1, 2, 4) and n % 32 == 0 and (T == 0 or kt.dtype == q.dtype)
    one = common                        # any text-tail length: a long one is taken in chunks
    split = common and bits == 1 and n > 0 and T <= 256
    return {cqb.CQ_PATH_FAST_ONE: one, cqb.CQ_PATH_FAST_SPLIT: split}.get(path, one or split)


def _run(K, V, q, kt, vt, bits, calib, path=cqb.CQ_PATH_AUTO, splits=0, out_dtype=None):
    import torch
    n = K.shape[2]
    kc, ks, km = cqb.cq_quantize_kv(K, bits, cqb.CQ_LAYOUT_K)
    vc, vs, vm = cqb.cq_quantize_kv(V, bits, cqb.CQ_LAYOUT_V)
    if path in FAST_PATHS and not fast_ok(q, K, kt, bits, path):
        with pytest.raises(cqb.CQError) as ei:
            cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=bits, sm_scale=SM, calib=calib,
                               path=path)
        assert ei.value.status == 2
        return None                     # the refusal is the checked result
    out = cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=bits, sm_scale=SM, calib=calib,
                             path=path, splits=splits, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out.float().cpu().numpy()


def _oracle(K, V, q, kt, vt, bits, calib, units=None):
    B, Hkv = K.shape[:2]
    Hq = q.shape[1]
    G = Hq // Hkv
    units = units or [(b, h) for b in range(B) for h in range(Hkv)]
    res = {}
    for b, h in units:
        res[(b, h)] = oracle_unit_decode(
            q[b, h * G:(h + 1) * G].cpu().numpy(), K[b, h].cpu().numpy(), V[b, h].cpu().numpy(),
            None if kt is None else kt[b, h].cpu().numpy(), None if vt is None else vt[b, h].cpu().numpy(),
            bits, SM, calib_f32(calib))
    return res


def _compare(got, ref, G, tol=REL_TOL):
    if got is None:                     # a forced path refused the shape (checked in _run)
        return 0.0
    worst = 0.0
    for (b, h), o in ref.items():
        worst = max(worst, rel_err(got[b, h * G:(h + 1) * G], o))
    assert worst <= tol, f"relative error {worst:.3e} > {tol}"
    return worst


@pytest.mark.parametrize("path", PATHS)
def test_tiny_fp32_single_head(path):
    K, V, q, _, _ = draw_inputs(1, 1, 1, 256, 0, dtype="float32", seed=1)
    note(f"decode tiny fp32 path={path}")
    got = _run(K, V, q, None, None, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, None, None, 1, RELATIVE), 1)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("calib", [None, RELATIVE, ABSOLUTE, IDENTITY])
@pytest.mark.parametrize("T", [0, 64])
@pytest.mark.parametrize("path", PATHS)
def test_gqa4_fp16(bits, calib, T, path):
    B, Hq, Hkv, n = 2, 8, 2, 800
    K, V, q, kt, vt = draw_inputs(B, Hq, Hkv, n, T, seed=11 + bits)
    note(f"decode B={B} Hq={Hq} Hkv={Hkv} n={n} T={T} bits={bits} calib={calib} path={path}")
    got = _run(K, V, q, kt, vt, bits, calib, path)
    _compare(got, _oracle(K, V, q, kt, vt, bits, calib), Hq // Hkv)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("n", [1, 31, 33, 1000])
@pytest.mark.parametrize("path", PATHS)
def test_group_sizes_and_ragged_lengths(G, n, path):
    Hkv, T = 2, 5
    K, V, q, kt, vt = draw_inputs(1, Hkv * G, Hkv, n, T, seed=G * 100 + n)
    note(f"decode G={G} n={n} T={T} path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), G)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 25])
def test_split_count_does_not_change_the_result(splits):
    import torch
    K, V, q, kt, vt = draw_inputs(1, 4, 1, 800, 64, seed=5)
    note(f"decode splits={splits}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, cqb.CQ_PATH_GENERIC, splits, out_dtype=torch.float32)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), 4)
    base = _run(K, V, q, kt, vt, 1, RELATIVE, cqb.CQ_PATH_GENERIC, 1, out_dtype=torch.float32)
    diff = float(np.max(np.abs(got - base)))
    assert diff <= 1e-5 * max(1.0, float(np.max(np.abs(base)))), f"max |diff| {diff:.3e}"


@pytest.mark.parametrize("path", PATHS)
def test_tail_only(path):
    import torch
    _, _, q, kt, vt = draw_inputs(2, 8, 2, 0, 16, seed=9)
    z = torch.zeros((2, 2, 128), dtype=torch.float32, device="cuda")
    note(f"decode n=0 T=16 path={path}")
    if path == cqb.CQ_PATH_FAST_SPLIT:
        with pytest.raises(cqb.CQError) as ei:
            cqb.cq_decode_attn(q, None, z, z, None, z, z, kt, vt, n=0, bits=1, sm_scale=SM, calib=RELATIVE,
                               path=path)
        assert ei.value.status == 2
        return
    out = cqb.cq_decode_attn(q, None, z, z, None, z, z, kt, vt, n=0, bits=1, sm_scale=SM, calib=RELATIVE,
                             path=path)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    for b in range(2):
        for hq in range(8):
            h = hq // 4
            ref = oracle.attend_dense(q[b, hq:hq + 1].cpu().numpy(), kt[b, h].cpu().numpy(),
                                      vt[b, h].cpu().numpy(), SM)
            assert rel_err(got[b, hq:hq + 1], ref) <= REL_TOL


@pytest.mark.parametrize("out_dtype", ["float16", "float32"])
@pytest.mark.parametrize("path", PATHS)
def test_fp32_query_tail_and_output(out_dtype, path):
    import torch
    K, V, q, kt, vt = draw_inputs(1, 8, 2, 320, 8, dtype="float32", seed=21)
    note(f"decode fp32 q/tail out={out_dtype} path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path, out_dtype=getattr(torch, out_dtype))
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), 4)


def test_oracle_packed_codes_decode():
    """Decode fed with codes and parameters packed by the oracle (isolates the decode kernels)."""
    import torch
    K, V, q, kt, vt = draw_inputs(2, 8, 2, 256, 64, seed=31)
    B, Hkv, n, d = K.shape
    kw, ks, km, kc = oracle.quantize(K.cpu().numpy(), 1, "K")
    vw, vs, vm, vc = oracle.quantize(V.cpu().numpy(), 1, "V")
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dt)
    note("decode from oracle-packed codes")
    for path in PATHS[:2]:
        out = cqb.cq_decode_attn(q, dev(kw.view(np.int32), torch.int32), dev(ks, torch.float32),
                                 dev(km, torch.float32), dev(vw.view(np.int32), torch.int32),
                                 dev(vs, torch.float32), dev(vm, torch.float32), kt, vt, n=n, bits=1,
                                 sm_scale=SM, calib=RELATIVE, path=path)
        torch.cuda.synchronize()
        ref = oracle.decode_attn(q.cpu().numpy(), kc, ks, km, vc, vs, vm, kt.cpu().numpy(), vt.cpu().numpy(),
                                 SM, calib_f32(RELATIVE))
        assert rel_err(out.float().cpu().numpy(), ref) <= REL_TOL


@pytest.mark.parametrize("path", PATHS)
def test_internvl_layer_sampled(path):
    """One InternVL-2.5-8B-shaped layer: B=16, 32q/8kv, n=3328, T=64, b=1, calibrated."""
    K, V, q, kt, vt = draw_inputs(16, 32, 8, 3328, 64, seed=2, host=False)
    note(f"decode internvl layer path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE, [(0, 0), (7, 5), (15, 7)]), 4)


@pytest.mark.parametrize("path", PATHS)
def test_long_context_sampled(path):
    """Headline shape: B=64, 32q/8kv, n=8192, T=64, b=1, calibrated, in the benchmark's launch."""
    K, V, q, kt, vt = draw_inputs(64, 32, 8, 8192, 64, seed=3, host=False)
    note(f"decode long context path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE, [(0, 0), (40, 2), (63, 7)]), 4)


@pytest.mark.parametrize("path", [cqb.CQ_PATH_AUTO, cqb.CQ_PATH_FAST])
def test_long_context_16k(path):
    """b = 1 at n = 16384 (128 key tiles, 16 per wave of the one-launch kernel)."""
    K, V, q, kt, vt = draw_inputs(2, 8, 2, 16384, 64, seed=15, host=False)
    note(f"decode n=16384 path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE, [(0, 1), (1, 0)]), 4)


@pytest.mark.parametrize("path", [cqb.CQ_PATH_AUTO, cqb.CQ_PATH_FAST_ONE])
def test_long_context_270k(path):
    """b = 1 at n = 270016 (2110 key tiles, about 264 per wave): each wave's
    int32 plane sums are moved into the 64-bit sums at least once on the way."""
    K, V, q, kt, vt = draw_inputs(1, 4, 1, 270016, 64, seed=16, host=False)
    note(f"decode n=270016 path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), 4)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_bit_width_sweep_sampled(bits):
    """Bit-width sweep shape (B=32, n=3328), calibration off, sampled units."""
    K, V, q, kt, vt = draw_inputs(32, 32, 8, 3328, 64, seed=4, host=False)
    note(f"decode bit sweep bits={bits}")
    got = _run(K, V, q, kt, vt, bits, None)
    _compare(got, _oracle(K, V, q, kt, vt, bits, None, [(0, 1), (31, 6)]), 4)


@pytest.mark.parametrize("n", [32, 96, 128, 1024, 1152, 2048, 2080, 4096, 4224, 8192, 12320])
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("path", [cqb.CQ_PATH_FAST_ONE, cqb.CQ_PATH_FAST_SPLIT])
def test_fast_kernel_tile_counts(n, G, path):
    """The one-launch kernel (tiles dealt to its 8 waves as they free up) at fewer tiles than waves,
    exactly one and several per wave, and the split kernels (1, 2, 4 and 8 tiles per wave) on both
    sides of each boundary, ragged tiles included."""
    K, V, q, kt, vt = draw_inputs(1, 2 * G, 2, n, 64, seed=n + G)
    note(f"decode fast n={n} G={G} path={path}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, path)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), G)


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 9, 64])
def test_split_chunk_counts(splits):
    """Split decode at requested chunk counts (each rounded to 4, 8, 16 or 32 tiles per chunk): every
    count agrees with the oracle and with every other count up to float32 summation order."""
    import torch
    K, V, q, kt, vt = draw_inputs(2, 8, 2, 2080, 64, seed=77)
    note(f"decode split chunks={splits}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, cqb.CQ_PATH_FAST_SPLIT, splits, out_dtype=torch.float32)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), 4)
    base = _run(K, V, q, kt, vt, 1, RELATIVE, cqb.CQ_PATH_FAST_SPLIT, 1, out_dtype=torch.float32)
    diff = float(np.max(np.abs(got - base)))
    assert diff <= 1e-5 * max(1.0, float(np.max(np.abs(base)))), f"max |diff| {diff:.3e}"


@pytest.mark.parametrize("n", [32, 160, 1152, 4224, 8192])
@pytest.mark.parametrize("splits", [1, 2, 4])
def test_split_tiles_per_wave(n, splits):
    """Few chunks per unit, so that every tiles-per-wave instantiation (up to 8) runs on short,
    ragged and long contexts, G = 4."""
    K, V, q, kt, vt = draw_inputs(1, 8, 2, n, 64, seed=n + 7 * splits)
    note(f"decode split n={n} chunks={splits}")
    got = _run(K, V, q, kt, vt, 1, RELATIVE, cqb.CQ_PATH_FAST_SPLIT, splits)
    _compare(got, _oracle(K, V, q, kt, vt, 1, RELATIVE), 4)


def test_split_workspace_reused_across_calls():
    """The split decode keeps its per-chunk partials in the workspace: three calls in a row on one
    workspace, the second smaller, each match the oracle."""
    import torch
    ws = torch.empty(cqb.lib.cq_decode_attn_workspace(4, 16, 4, 4096, 64, 128, 1), dtype=torch.uint8,
                     device="cuda")
    for (B, n, seed) in [(4, 4096, 81), (2, 1024, 82), (4, 4096, 83)]:
        K, V, q, kt, vt = draw_inputs(B, 16, 4, n, 64, seed=seed)
        kc, ks, km = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
        vc, vs, vm = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
        note(f"decode split reused workspace B={B} n={n}")
        out = cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=1, sm_scale=SM, calib=RELATIVE,
                                 workspace=ws, path=cqb.CQ_PATH_FAST_SPLIT)
        torch.cuda.synchronize()
        _compare(out.float().cpu().numpy(), _oracle(K, V, q, kt, vt, 1, RELATIVE), 4)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("n", [32, 96, 1056, 3328])
def test_fast_kernel_multibit(bits, G, n):
    """Matrix-core kernels for b = 2, 4, 8: tiles of 128/b tokens, half-filled last tiles, tail."""
    K, V, q, kt, vt = draw_inputs(1, 2 * G, 2, n, 64, seed=bits * 1000 + n + G)
    note(f"decode fast bits={bits} n={n} G={G}")
    got = _run(K, V, q, kt, vt, bits, None, cqb.CQ_PATH_FAST)
    _compare(got, _oracle(K, V, q, kt, vt, bits, None), G)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_fast_kernel_multibit_fp32_and_calibrated(bits):
    import torch
    K, V, q, kt, vt = draw_inputs(1, 8, 2, 320, 8, dtype="float32", seed=77 + bits)
    note(f"decode fast bits={bits} fp32 calibrated")
    got = _run(K, V, q, kt, vt, bits, RELATIVE, cqb.CQ_PATH_FAST, out_dtype=torch.float32)
    _compare(got, _oracle(K, V, q, kt, vt, bits, RELATIVE), 4)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("n", [1024, 3328, 7040, 8192])
def test_one_unit_per_cu_instance_equals_two_per_cu(bits, n):
    """b = 2, 4, 8 at most one (batch, kv head) unit per CU (here 32 sequences
    of 8 kv heads) keep the scores of the first 6912 tokens in LDS, so only
    the key tiles past them are read twice; more units than CUs (40
    sequences) keep fewer (1792 / 2112 / 2240 tokens at b = 2 / 4 / 8) on
    caches shorter than 4096 tokens (6144 at b = 2), and the same 6912 on
    longer ones.  The scores are the same either way, so the first 32
    sequences of the larger batch must equal the smaller batch bit for bit,
    and the oracle within 2e-3."""
    import torch
    K, V, q, kt, vt = draw_inputs(40, 32, 8, n, 64, seed=90 + bits + n, host=False)
    note(f"decode kept-score instances bits={bits} n={n}")
    big = _run(K, V, q, kt, vt, bits, None)
    small = _run(*(x[:32].contiguous() for x in (K, V, q, kt, vt)), bits, None)
    assert np.array_equal(big[:32], small)
    _compare(small, _oracle(K[:32], V[:32], q[:32], kt[:32], vt[:32], bits, None, [(0, 0), (31, 7)]), 4)
