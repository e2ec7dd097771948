"""GPU quantization vs the oracle: codes, packed words, scale and min must be
bit-exact (QbitAI article on CalibQuant, "Method" part 1)."""
import numpy as np
import pytest

import oracle
from helpers import draw_inputs, note, words_u32

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")
PATHS = [cqb.CQ_PATH_GENERIC, cqb.CQ_PATH_AUTO, cqb.CQ_PATH_FAST]
LAYOUTS = {cqb.CQ_LAYOUT_K: "K", cqb.CQ_LAYOUT_V: "V"}


# one (batch, head) of the fused kernel spans at most this many tokens on a
# 256-CU MI355X: 512-token chunks, all resident at once, 2 workgroups per CU
FUSED_MAX_N = 512 * 512


def _fast_ok(x_dev, bits):
    import torch
    return x_dev.dtype == torch.float16 and bits == 1 and 1 <= x_dev.shape[2] <= FUSED_MAX_N


def _check_units(x_dev, bits, layout, path, units=None):
    import torch
    B, H, n, d = x_dev.shape
    note(f"quantize shape={tuple(x_dev.shape)} dtype={x_dev.dtype} bits={bits} layout={LAYOUTS[layout]} path={path}")
    if path == cqb.CQ_PATH_FAST and not _fast_ok(x_dev, bits):
        with pytest.raises(cqb.CQError) as ei:
            cqb.cq_quantize_kv(x_dev, bits, layout, path=path)
        assert ei.value.status == 2          # CQ_ERR_UNSUPPORTED, nothing enqueued
        return
    ws = torch.full((cqb.lib.cq_quantize_kv_workspace(B, H, n, d, bits),), 7, dtype=torch.uint8, device="cuda")
    codes, scale, minv = cqb.cq_quantize_kv(x_dev, bits, layout, path=path, workspace=ws)
    torch.cuda.synchronize()
    if path != cqb.CQ_PATH_GENERIC and _fast_ok(x_dev, bits):
        assert int(ws[:4].view(torch.int32).item()) == 0, "cooperative wait timed out"
    B, H = x_dev.shape[:2]
    units = units or [(b, h) for b in range(B) for h in range(H)]
    for b, h in units:
        xu = x_dev[b, h].cpu().numpy()
        c, sc, mn, _ = oracle.quantize_unit(xu, bits)
        ref_words = oracle.pack(c, bits, LAYOUTS[layout])
        got = words_u32(codes[b, h])
        assert got.shape == ref_words.shape
        bad = np.argwhere(got != ref_words)
        assert bad.size == 0, f"unit {(b, h)}: {len(bad)} words differ, first at {bad[:3].tolist()}"
        assert np.array_equal(scale[b, h].cpu().numpy().view(np.uint32), sc.view(np.uint32)), f"scale {(b, h)}"
        assert np.array_equal(minv[b, h].cpu().numpy(), mn), f"min {(b, h)}"      # -0 == +0


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("path", PATHS)
def test_tiny_fp32_single_head(layout, path):
    K, V, *_ = draw_inputs(1, 1, 1, 256, 0, dtype="float32", seed=1)
    _check_units(K, 1, layout, path)
    _check_units(V, 1, layout, path)


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("n", [1, 45, 800, 1000])
@pytest.mark.parametrize("path", PATHS)
def test_fp16_ragged(bits, layout, n, path):
    K, *_ = draw_inputs(2, 2, 2, n, 0, seed=7 + n)
    _check_units(K, bits, layout, path)


@pytest.mark.parametrize("bits", [1, 2, 8])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("path", PATHS)
def test_forced_ties_and_degenerate(bits, dtype, path):
    import torch
    L = (1 << bits) - 1
    n, d = 96, 128
    rng = np.random.default_rng(bits)
    x = np.empty((n, d))
    for j in range(d):
        mn = float(rng.integers(-8, 8))
        step = 2.0 ** -int(rng.integers(0, 4))
        k = rng.integers(0, L + 1, n).astype(np.float64)
        half = rng.random(n) < 0.5
        k[half] = np.minimum(k[half], L - 1) + 0.5           # exact half-levels
        k[0], k[1] = 0, L
        x[:, j] = mn + k * step
    x[:, 5] = 3.0                                            # constant channel
    x[:, 9] = -0.0
    x[3, 9] = 0.0
    xd = torch.from_numpy(x.astype(dtype)).reshape(1, 1, n, d).cuda()
    for layout in (0, 1):
        _check_units(xd, bits, layout, path)


@pytest.mark.parametrize("path", PATHS[:2])
def test_empty_cache(path):
    import torch
    x = torch.empty((2, 3, 0, 128), dtype=torch.float16, device="cuda")
    note("quantize n=0")
    codes, scale, minv = cqb.cq_quantize_kv(x, 1, 0, path=path)
    torch.cuda.synchronize()
    assert codes.numel() == 0 and (scale == 0).all() and (minv == 0).all()


@pytest.mark.parametrize("path", PATHS)
def test_internvl_layer_sampled_units(path):
    """Full one-layer InternVL-2.5-8B shape (B=16, 8 kv heads, n=3328), sampled units."""
    K, V, *_ = draw_inputs(16, 32, 8, 3328, 0, seed=2, host=False)
    units = [(0, 0), (5, 3), (15, 7)]
    _check_units(K, 1, 0, path, units)
    _check_units(V, 1, 1, path, units)


@pytest.mark.parametrize("path", PATHS)
def test_long_context_sampled_units(path):
    """Headline shape (B=64, 8 kv heads, n=8192, fp16), in the launch the benchmark times."""
    K, V, *_ = draw_inputs(64, 32, 8, 8192, 0, seed=3, host=False)
    units = [(0, 0), (31, 4), (63, 7)]
    _check_units(K, 1, 0, path, units)
    _check_units(V, 1, 1, path, units)


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("path", PATHS)
def test_longer_than_one_fused_round(layout, path):
    """n = 270016 has more 512-token chunks per head (528) than the device
    holds workgroups: AUTO takes the generic kernels, FAST is refused."""
    x, _, _, _, _ = draw_inputs(1, 4, 1, 270016, 0, seed=17, host=False)
    _check_units(x, 1, layout, path)


def test_fused_repeated_launches_are_identical():
    """The fused kernel's rendezvous state is re-initialised by every call."""
    import torch
    K, *_ = draw_inputs(8, 32, 8, 1000, 0, seed=13, host=False)
    note("quantize fused x5")
    ref = [t.clone() for t in cqb.cq_quantize_kv(K, 1, 0, path=cqb.CQ_PATH_FAST)]
    ws = torch.empty((cqb.lib.cq_quantize_kv_workspace(8, 8, 1000, 128, 1),), dtype=torch.uint8, device="cuda")
    for _ in range(5):
        got = cqb.cq_quantize_kv(K, 1, 0, path=cqb.CQ_PATH_FAST, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
