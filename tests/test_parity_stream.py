"""Chunked-prefill quantization on the GPU against the oracle (QbitAI article
on CalibQuant, "Method" part 1: per-channel range over one head's tokens,
uniform rounding to the nearest level).

* cq_kv_range_update: the merged range and the grew flags equal the
  oracle's range_update chunk by chunk (values exact, zeros stored as +0);
* cq_quantize_kv_rows: the words of the coded rows, scale and minimum equal
  the oracle's quantize_with_range on the same given range, bit for bit, and
  nothing outside the rows (or in masked units) is written;
* the chunked prefill (deferred and eager) ends bit for bit at
  cq_quantize_kv's one-shot codes, also at the long-context shape.
"""
import numpy as np
import pytest

import oracle
from helpers import note, words_u32
from workloads import ROLE_K, ROLE_V, kv_torch

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")
from extreme_bit_kv_amd.prefill import ChunkedVisualQuantizer  # noqa: E402

LAYOUTS = {cqb.CQ_LAYOUT_K: "K", cqb.CQ_LAYOUT_V: "V"}
SENTINEL = 0x5A5A5A5A


def _cache(B, H, rows, seg, dtype, seed, role=ROLE_K):
    """A cache of `rows` rows per unit whose first `seg` rows hold the
    synthetic visual tokens; the rows after them hold 1000 (any read of them
    would show in a range)."""
    import torch
    x = kv_torch(seed, 0, role, B, H, rows, 128, dtype, "cuda")
    x[:, :, seg:] = 1000.0
    return x


def _ranges(x_np, seed):
    rng = np.random.default_rng(seed)
    lo = x_np.min(axis=0).astype(np.float32)
    hi = x_np.max(axis=0).astype(np.float32)
    w = hi - lo
    odd_lo, odd_hi = lo.copy(), hi.copy()
    odd_hi[0] = odd_lo[0]
    odd_lo[1], odd_hi[1] = hi[1], lo[1]
    odd_lo[2] = odd_hi[2] = np.float32(rng.standard_normal())
    odd_lo[3] = np.float32(lo[3] - np.float32(2.0 ** -20))      # off the float16 grid
    return {"own": (lo, hi), "narrow": (lo + np.float32(0.3) * w, hi - np.float32(0.25) * w),
            "wide": (lo - np.float32(0.5) * w, hi + np.float32(0.125) * w), "odd": (odd_lo, odd_hi)}


@pytest.mark.parametrize("dtype", ["float16", "float32"])
@pytest.mark.parametrize("cuts", [[0, 512, 1024], [0, 1, 33, 300, 700, 1024], [0, 1024]])
def test_range_update_matches_oracle(dtype, cuts):
    import torch
    B, H, rows, n = 2, 4, 1280, 1024
    x = _cache(B, H, rows, n, dtype, seed=3)
    x[:, :, 700:1024] = x[:, :, 0:324].clone()                # a chunk that widens nothing ...
    x[1, 2, 800, 5] = -500.0                                  # ... except in one unit
    note(f"range update dtype={dtype} cuts={cuts}")
    xs = x.cpu().numpy()
    mn = mx = None
    ref = {}
    grew = torch.full((B, H), 7, dtype=torch.int32, device="cuda")
    for a, b in zip(cuts[:-1], cuts[1:]):
        mn, mx = cqb.cq_kv_range_update(x, a, b - a, mn, mx, reset=a == 0, grew=grew)
        torch.cuda.synchronize()
        g = grew.cpu().numpy()
        for u in range(B * H):
            bb, hh = divmod(u, H)
            prev = ref.get(u, (None, None))
            lo, hi, gr = oracle.range_update(prev[0], prev[1], xs[bb, hh, a:b], reset=a == 0)
            ref[u] = (lo, hi)
            assert np.array_equal(mn[bb, hh].cpu().numpy(), lo), f"min, unit {u}, chunk {a}"
            assert np.array_equal(mx[bb, hh].cpu().numpy(), hi), f"max, unit {u}, chunk {a}"
            assert int(g[bb, hh]) == int(gr), f"grew, unit {u}, chunk {a}"
    for t in (mn, mx):
        bits = t.cpu().numpy().view(np.uint32)
        assert not np.any(bits == 0x80000000), "a zero stored as -0"
    if cuts == [0, 512, 1024]:
        assert grew.cpu().numpy()[1, 2] == 1


@pytest.mark.parametrize("bits", [1, 2, 4, 8])
@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("dtype", ["float16", "float32"])
def test_rows_on_given_range(bits, layout, dtype):
    import torch
    B, H, rows, n = 2, 3, 1600, 1536
    t0, m = (512, 640) if dtype == "float16" else (512, 160)  # 1.25 tiles of 512; several generic blocks
    x = _cache(B, H, rows, n, dtype, seed=10 + bits)
    xs = x.cpu().numpy()
    E = 32 // bits
    mask = torch.ones((B, H), dtype=torch.int32, device="cuda")
    mask[1, 1] = 0
    for name, (lo, hi) in _ranges(xs[0, 0, :n], bits).items():
        note(f"rows on a given range: bits={bits} layout={LAYOUTS[layout]} dtype={dtype} range={name}")
        mn = torch.from_numpy(np.broadcast_to(lo, (B, H, 128)).copy()).cuda()
        mx = torch.from_numpy(np.broadcast_to(hi, (B, H, 128)).copy()).cuda()
        shape = cqb.code_words_shape(B, H, n, 128, bits, layout)
        codes = torch.full(shape, SENTINEL, dtype=torch.int32, device="cuda")
        scale = torch.full((B, H, 128), -7.0, device="cuda")
        minv = torch.full((B, H, 128), -7.0, device="cuda")
        cqb.cq_quantize_kv_rows(x, t0, m, bits, layout, mn, mx, n, codes, scale, minv, unit_mask=mask)
        torch.cuda.synchronize()
        for bb in range(B):
            for hh in range(H):
                got = words_u32(codes[bb, hh])
                if mask[bb, hh].item() == 0:
                    assert np.all(got == SENTINEL) and np.all(scale[bb, hh].cpu().numpy() == -7.0)
                    continue
                c, sc, mv = oracle.quantize_with_range(xs[bb, hh, t0:t0 + m], lo, hi, bits)
                if layout == cqb.CQ_LAYOUT_K:
                    ref = oracle.pack(c, bits, "K")                    # [W, m]
                    win, rest = got[:, t0:t0 + m], np.delete(got, np.s_[t0:t0 + m], axis=1)
                else:
                    ref = oracle.pack(c, bits, "V")                    # [m/E, d]
                    win, rest = got[t0 // E:(t0 + m) // E], np.delete(got, np.s_[t0 // E:(t0 + m) // E], axis=0)
                bad = np.argwhere(win != ref)
                assert bad.size == 0, f"unit {(bb, hh)}: {len(bad)} words differ, first {bad[:3].tolist()}"
                assert np.all(rest == SENTINEL), "a word outside the rows was written"
                assert np.array_equal(scale[bb, hh].cpu().numpy().view(np.uint32), sc.view(np.uint32))
                assert np.array_equal(minv[bb, hh].cpu().numpy(), mv)


def _one_shot(x_seg, bits, layout):
    return cqb.cq_quantize_kv(x_seg.contiguous(), bits, layout)


@pytest.mark.parametrize("bits", [1, 2])
@pytest.mark.parametrize("eager", [False, True])
def test_chunked_prefill_equals_one_shot(bits, eager):
    """A segment at row 96 of a 2200-row cache, 2000 tokens in chunks of
    512, 512, 512, 464 (the last one ragged)."""
    import torch
    B, H, rows, row0, n = 2, 8, 2200, 96, 2000
    k = _cache(B, H, rows, rows, "float16", seed=21, role=ROLE_K)
    v = _cache(B, H, rows, rows, "float16", seed=21, role=ROLE_V)
    k[:, :, :row0] = -1000.0
    k[:, :, row0 + n:] = 1000.0
    v[:, :, :row0] = -1000.0
    note(f"chunked prefill bits={bits} eager={eager}")
    q = ChunkedVisualQuantizer(k, v, n, bits=bits, row0=row0, eager=eager)
    for m in (512, 512, 512, 464):
        q.append(m)
    cache = q.finish()
    torch.cuda.synchronize()
    for L, x, got in ((cqb.CQ_LAYOUT_K, k, cache.k), (cqb.CQ_LAYOUT_V, v, cache.v)):
        want = _one_shot(x[:, :, row0:row0 + n], bits, L)
        torch.cuda.synchronize()
        for g, w, what in zip(got, want, ("codes", "scale", "min")):
            assert torch.equal(g, w), f"{LAYOUTS[L]} {what} differs from the one-shot quantization"
        xs = x[1, 5, row0:row0 + n].cpu().numpy()
        c, sc, mv, _ = oracle.quantize_unit(xs, bits)
        assert np.array_equal(words_u32(got[0][1, 5]), oracle.pack(c, bits, LAYOUTS[L]))


def test_eager_codes_follow_the_segment():
    """After every eager append the codes are those of the segment so far
    (coded on its own range), in the final layout."""
    import torch
    B, H, n = 1, 4, 1536
    k = _cache(B, H, n, n, "float16", seed=5)
    v = _cache(B, H, n, n, "float16", seed=6, role=ROLE_V)
    k[0, 3, 1200, 7] = 60.0                                   # the last chunk widens one unit
    q = ChunkedVisualQuantizer(k, v, n, bits=1, eager=True)
    note("eager chunked prefill, per-chunk check")
    ks = k.cpu().numpy()
    for t in (0, 512, 1024):
        q.append(512)
        torch.cuda.synchronize()
        codes = q.out[cqb.CQ_LAYOUT_K][0]
        for h in range(H):
            c, _, _, _ = oracle.quantize_unit(ks[0, h, :t + 512], 1)
            got = words_u32(codes[0, h])[:, :t + 512]
            assert np.array_equal(got, oracle.pack(c, 1, "K")), f"after rows {t + 512}, head {h}"
    assert q.grew[cqb.CQ_LAYOUT_K].cpu().numpy()[0, 3] == 1


def test_long_context_chunked_prefill():
    """The long-context shape (64 sequences x 8 kv heads, 8192 visual tokens,
    512-token chunks): the chunked prefill equals the one-shot quantization
    for every unit, and the oracle on sampled units."""
    import torch
    B, H, n = 64, 8, 8192
    note("long-context chunked prefill B=64 H=8 n=8192")
    k = kv_torch(7, 0, ROLE_K, B, H, n, 128, "float16", "cuda")
    v = kv_torch(7, 0, ROLE_V, B, H, n, 128, "float16", "cuda")
    q = ChunkedVisualQuantizer(k, v, n, bits=1)
    for _ in range(n // 512):
        q.append(512)
    cache = q.finish()
    for L, x, got in ((cqb.CQ_LAYOUT_K, k, cache.k), (cqb.CQ_LAYOUT_V, v, cache.v)):
        want = _one_shot(x, 1, L)
        torch.cuda.synchronize()
        for g, w in zip(got, want):
            assert torch.equal(g, w)
        for bb, hh in ((0, 0), (37, 5), (63, 7)):
            c, sc, mv, _ = oracle.quantize_unit(x[bb, hh].cpu().numpy(), 1)
            assert np.array_equal(words_u32(got[0][bb, hh]), oracle.pack(c, 1, LAYOUTS[L]))
            assert np.array_equal(got[1][bb, hh].cpu().numpy().view(np.uint32), sc.view(np.uint32))
