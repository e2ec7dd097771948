"""cq_quantize_kv_pair on the GPU: the outputs of two cq_quantize_kv calls (K
layout for k, V layout for v) bit for bit, and the oracle's (QbitAI article
on CalibQuant, "Method" part 1: channel-wise quantization of K and of V)."""
import numpy as np
import pytest

import oracle
from helpers import draw_inputs, note, words_u32

pytestmark = pytest.mark.gpu

cqb = pytest.importorskip("extreme_bit_kv_amd")


def _pair_vs_single(k, v, bits, path=cqb.CQ_PATH_AUTO, ws_fill=None):
    import torch
    B, H, n, d = k.shape
    ws = None
    if ws_fill is not None:
        ws = torch.full((cqb.lib.cq_quantize_kv_pair_workspace(B, H, n, d, bits),), ws_fill, dtype=torch.uint8,
                        device="cuda")
    (kc, ks, km), (vc, vs, vm) = cqb.cq_quantize_kv_pair(k, v, bits, workspace=ws, path=path)
    k1 = cqb.cq_quantize_kv(k, bits, cqb.CQ_LAYOUT_K)
    v1 = cqb.cq_quantize_kv(v, bits, cqb.CQ_LAYOUT_V)
    torch.cuda.synchronize()
    for got, want, what in zip((kc, ks, km, vc, vs, vm), (*k1, *v1), ("k codes", "k scale", "k min", "v codes",
                                                                          "v scale", "v min")):
        assert torch.equal(got, want), f"{what} differ from the single-tensor call"
    if ws is not None:
        assert int(ws[:4].view(torch.int32).item()) == 0, "a wait timed out"
    return (kc, ks, km), (vc, vs, vm)


@pytest.mark.parametrize("n", [1, 31, 512, 513, 1000, 3328])
@pytest.mark.parametrize("B,H", [(1, 1), (3, 8)])
def test_fused_pair_equals_two_calls(n, B, H):
    K, V, *_ = draw_inputs(B, 4 * H, H, n, 0, seed=n + B, host=False)
    note(f"quantize pair fp16 b=1 B={B} H={H} n={n}")
    (kc, ks, km), (vc, vs, vm) = _pair_vs_single(K, V, 1, ws_fill=7)
    b, h = B - 1, H - 1
    for x, words, layout in ((K, kc, "K"), (V, vc, "V")):
        c, sc, mn, _ = oracle.quantize_unit(x[b, h].cpu().numpy(), 1)
        assert np.array_equal(words_u32(words[b, h]), oracle.pack(c, 1, layout))


@pytest.mark.parametrize("bits,dtype", [(2, "float16"), (8, "float16"), (1, "float32"), (4, "float32")])
def test_pair_one_tensor_after_the_other(bits, dtype):
    """Shapes the fused kernel does not take: the two tensors in turn."""
    K, V, *_ = draw_inputs(2, 8, 2, 700, 0, dtype=dtype, seed=bits, host=False)
    note(f"quantize pair bits={bits} dtype={dtype}")
    _pair_vs_single(K, V, bits)


def test_pair_paths():
    import torch
    K, V, *_ = draw_inputs(2, 8, 2, 1024, 0, seed=5, host=False)
    _pair_vs_single(K, V, 1, path=cqb.CQ_PATH_GENERIC)
    _pair_vs_single(K, V, 1, path=cqb.CQ_PATH_FAST)
    K2, V2, *_ = draw_inputs(2, 8, 2, 1024, 0, seed=5, host=False)
    with pytest.raises(cqb.CQError) as ei:
        cqb.cq_quantize_kv_pair(K2.float().contiguous(), V2.float().contiguous(), 1, path=cqb.CQ_PATH_FAST)
    assert ei.value.status == 2
    torch.cuda.synchronize()


def test_pair_repeated_on_one_workspace():
    """The word reset runs in every call: a workspace left by a call serves the next."""
    import torch
    K, V, *_ = draw_inputs(4, 16, 4, 2048, 0, seed=11, host=False)
    ws = torch.empty(cqb.lib.cq_quantize_kv_pair_workspace(4, 4, 2048, 128, 1), dtype=torch.uint8, device="cuda")
    first = cqb.cq_quantize_kv_pair(K, V, 1, workspace=ws)
    first = [t.clone() for part in first for t in part]
    for _ in range(3):
        again = cqb.cq_quantize_kv_pair(K, V, 1, workspace=ws)
        torch.cuda.synchronize()
        for a, b_ in zip(first, (t for part in again for t in part)):
            assert torch.equal(a, b_)


def test_pair_long_context_headline():
    """The long-context shape (64 x 8 units, n = 8192) in one launch."""
    K, V, *_ = draw_inputs(64, 32, 8, 8192, 0, seed=3, host=False)
    note("quantize pair long context")
    (kc, ks, km), (vc, vs, vm) = _pair_vs_single(K, V, 1, ws_fill=3)
    for b, h in ((0, 0), (63, 7)):
        for x, words, layout in ((K, kc, "K"), (V, vc, "V")):
            c, sc, mn, _ = oracle.quantize_unit(x[b, h].cpu().numpy(), 1)
            assert np.array_equal(words_u32(words[b, h]), oracle.pack(c, 1, layout))


@pytest.mark.parametrize("B,H,n", [(64, 8, 1000), (32, 8, 3328)])
def test_pair_several_rounds_ragged(B, H, n):
    """More items than workgroups and a ragged last chunk: workgroups walk
    several items each, the K items hand over to V items inside a workgroup,
    and the half of a next item requested during a rendezvous includes
    rows clamped at the segment's end."""
    K, V, *_ = draw_inputs(B, 4 * H, H, n, 0, seed=n + 17, host=False)
    note(f"quantize pair several rounds B={B} H={H} n={n}")
    (kc, ks, km), (vc, vs, vm) = _pair_vs_single(K, V, 1, ws_fill=9)
    for b, h in ((0, 1), (B // 2, 3), (B - 1, H - 1)):
        for x, words, scale, layout in ((K, kc, ks, "K"), (V, vc, vs, "V")):
            c, sc, mn, _ = oracle.quantize_unit(x[b, h].cpu().numpy(), 1)
            assert np.array_equal(words_u32(words[b, h]), oracle.pack(c, 1, layout))
            assert np.array_equal(scale[b, h].cpu().numpy().view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("pair", [True, False])
def test_wait_time_out_is_reported(pair):
    """A fused call whose workgroups give up waiting (forced from the host
    with cq_opts.max_polls = 1: every kernel still exits normally) raises
    CQ_ERR_TIMEOUT through cq_quantize_status, and the header word that
    collects time-outs keeps the record; the next call with the default
    bound clears the call's status word and is exact again."""
    import torch
    B, H, n = 16, 8, 8192                        # 16 chunks per (batch, head): every head has waits
    K, V, *_ = draw_inputs(B, 4 * H, H, n, 0, seed=91, host=False)
    size = (cqb.lib.cq_quantize_kv_pair_workspace if pair else cqb.lib.cq_quantize_kv_workspace)(B, H, n, 128, 1)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")

    def call(**kw):
        if pair:
            return cqb.cq_quantize_kv_pair(K, V, 1, workspace=ws, **kw)[0]
        return cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K, workspace=ws, **kw)

    note(f"quantize forced time-out pair={pair}")
    with pytest.raises(cqb.CQError) as ei:
        call(check=True, max_polls=1)
    assert ei.value.status == cqb.CQ_ERR_TIMEOUT
    assert int(ws[4:8].view(torch.int32).item()) == 1
    note(f"quantize after a time-out pair={pair}")
    kc, ks, km = call(check=True)                # raises if any wait gave up
    assert int(ws[:4].view(torch.int32).item()) == 0
    assert int(ws[4:8].view(torch.int32).item()) == 1      # the collected record stays
    kw, kso, kmo, _ = oracle.quantize(K[5:6, 3:4].cpu().numpy(), 1, "K")
    assert np.array_equal(words_u32(kc[5:6, 3:4]), kw)
    assert np.array_equal(ks[5:6, 3:4].cpu().numpy(), kso) and np.array_equal(km[5:6, 3:4].cpu().numpy(), kmo)


def test_generic_path_reports_no_time_out():
    """Float32 input runs K and V one after the other through the generic
    kernels on one workspace (the fused launch takes float16 only).  They
    never wait, so the status words stay 0 whatever the poll limit."""
    import torch
    K, V, *_ = draw_inputs(2, 8, 2, 1024, 0, dtype="float32", seed=92, host=False)
    ws = torch.zeros(cqb.lib.cq_quantize_kv_pair_workspace(2, 2, 1024, 128, 1), dtype=torch.uint8, device="cuda")
    note("quantize pair fp32 with a poll limit")
    cqb.cq_quantize_kv_pair(K, V, 1, workspace=ws, check=True, max_polls=1)
    assert int(ws[4:8].view(torch.int32).item()) == 0
