"""The C-ABI library loads, exports every entry point include/cq.h declares,
and rejects invalid arguments before touching the GPU (no GPU needed: only
validation paths are exercised, and they return before any HIP call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

cqb = pytest.importorskip("extreme_bit_kv_amd", reason="libcq.so not built")
lib = cqb.lib

FAKE = ctypes.c_void_p(0x10000)       # never dereferenced: every call below fails validation
ODD = ctypes.c_void_p(0x10008)        # 8-byte aligned only: bulk buffers must be 16-byte aligned


def _declared():
    text = open(os.path.join(ROOT, "include", "cq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*]+\s+)+\**(cq_\w+)\s*\(", text, re.M)))


def test_header_and_exports_agree():
    decl = _declared()
    assert decl and set(decl) == set(cqb.EXPORTED)
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    assert lib.cq_abi_version() == 3
    for s in range(6):
        assert lib.cq_status_str(s)
    assert b"TIMEOUT" in lib.cq_status_str(5)
    assert b"unknown" in lib.cq_status_str(99)


def test_workspace_queries():
    assert lib.cq_quantize_kv_workspace(64, 8, 8192, 128, 1) > 0
    assert lib.cq_quantize_kv_workspace(1, 1, 256, 128, 3) == 0          # bad bits
    assert lib.cq_decode_attn_workspace(16, 32, 8, 3328, 64, 128, 1) > 0
    assert lib.cq_decode_attn_workspace(16, 30, 8, 3328, 64, 128, 1) == 0  # Hq % Hkv
    assert lib.cq_decode_attn_fp16_workspace(4, 32, 8, 3392, 128) > 0
    assert lib.cq_decode_attn_fp16_workspace(4, 32, 8, 0, 128) == 0


def _quant(**kw):
    a = dict(x=FAKE, dt=cqb.CQ_F16, B=1, H=1, n=64, d=128, bits=1, layout=cqb.CQ_LAYOUT_K, codes=FAKE,
             scale=FAKE, minv=FAKE, ws=FAKE, wsb=1 << 30, opts=None)
    a.update(kw)
    return lib.cq_quantize_kv(a["x"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["bits"], a["layout"],
                              a["codes"], a["scale"], a["minv"], a["ws"], a["wsb"], a["opts"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scale=None), 1), (dict(minv=None), 1),
    (dict(bits=3), 1), (dict(bits=0), 1), (dict(dt=7), 1), (dict(layout=2), 1), (dict(n=-1), 1),
    (dict(B=-1), 1), (dict(d=48, bits=1), 1), (dict(d=64), 2), (dict(d=256), 2),
    (dict(ws=None), 3), (dict(wsb=16), 3),
    (dict(opts=ctypes.pointer(cqb.cq_opts(9, 0))), 1),
    (dict(x=ODD), 1), (dict(codes=ODD), 1), (dict(ws=ODD), 1), (dict(scale=ctypes.c_void_p(0x10002)), 1),
])
def test_quantize_rejects(kw, status):
    assert _quant(**kw) == status


def _decode(**kw):
    a = dict(q=FAKE, qdt=0, kc=FAKE, ks=FAKE, km=FAKE, vc=FAKE, vs=FAKE, vm=FAKE, kt=FAKE, vt=FAKE, tdt=0,
             B=2, Hq=32, Hkv=8, n=64, T=8, d=128, bits=1, sm=0.088, calib=None, out=FAKE, odt=0,
             ws=FAKE, wsb=1 << 30, opts=None)
    a.update(kw)
    return lib.cq_decode_attn(a["q"], a["qdt"], a["kc"], a["ks"], a["km"], a["vc"], a["vs"], a["vm"], a["kt"],
                              a["vt"], a["tdt"], a["B"], a["Hq"], a["Hkv"], a["n"], a["T"], a["d"], a["bits"],
                              a["sm"], a["calib"], a["out"], a["odt"], a["ws"], a["wsb"], a["opts"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(kc=None), 1), (dict(vs=None), 1), (dict(kt=None), 1),
    (dict(T=0), 1),                                   # tails given but T == 0
    (dict(n=0, T=0, kt=None, vt=None), 1),            # nothing to attend over
    (dict(Hq=30), 1), (dict(Hkv=0), 1), (dict(bits=5), 1), (dict(qdt=3), 1), (dict(odt=3), 1),
    (dict(tdt=2), 1), (dict(sm=float("nan")), 1), (dict(d=64), 2), (dict(Hq=80, Hkv=8), 2),
    # the workspace cases force the split-K path, the one that needs a workspace
    (dict(ws=None, opts=ctypes.pointer(cqb.cq_opts(1, 0))), 3),
    (dict(wsb=8, opts=ctypes.pointer(cqb.cq_opts(1, 0))), 3),
    (dict(opts=ctypes.pointer(cqb.cq_opts(0, -2))), 1),
    (dict(opts=ctypes.pointer(cqb.cq_opts(2, 0)), Hq=64), 2),      # matrix-core path: group sizes 1, 2, 4
    (dict(opts=ctypes.pointer(cqb.cq_opts(8, 0))), 1),              # no such path
    (dict(opts=ctypes.pointer(cqb.cq_opts(5, 0)), bits=2), 2),     # LDS-score schedule: b = 1 only ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(5, 0)), n=8320), 2),     # ... and G x ceil(n/128) <= 256
    (dict(opts=ctypes.pointer(cqb.cq_opts(5, 0)), Hq=24), 2),      # ... and G in 1, 2, 4
    (dict(opts=ctypes.pointer(cqb.cq_opts(6, 0)), bits=2), 2),     # pipelined schedule: b = 1 only ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(6, 0)), n=8224), 2),     # ... 32 <= n <= 8192 ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(6, 0)), n=0, kc=None, vc=None), 2),
    (dict(opts=ctypes.pointer(cqb.cq_opts(6, 0)), T=129), 2),      # ... T <= 128 ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(6, 0)), n=80), 2),       # ... n a multiple of 32
    (dict(opts=ctypes.pointer(cqb.cq_opts(6, 0)), Hq=48), 2),      # ... G in 1, 2, 4
    (dict(opts=ctypes.pointer(cqb.cq_opts(7, 0)), bits=2), 2),     # all-in-flight schedule: b = 1 only ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(7, 0)), n=4128), 2),     # ... n <= 4096 ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(7, 0)), T=257), 2),      # ... T <= 256 ...
    (dict(opts=ctypes.pointer(cqb.cq_opts(7, 0)), n=80), 2),       # ... n a multiple of 32
    (dict(opts=ctypes.pointer(cqb.cq_opts(7, 0)), Hq=48), 2),      # ... G in 1, 2, 4
    (dict(opts=ctypes.pointer(cqb.cq_opts(3, 0)), Hq=64), 2),      # one-launch schedule: group sizes 1, 2, 4
    (dict(opts=ctypes.pointer(cqb.cq_opts(4, 0)), bits=2), 2),     # split schedule: b = 1 only
    (dict(opts=ctypes.pointer(cqb.cq_opts(4, 0)), n=0, kc=None, vc=None), 2),   # ... and n > 0
    (dict(opts=ctypes.pointer(cqb.cq_opts(4, 0)), n=96, ws=None), 3),           # it needs a workspace
    (dict(opts=ctypes.pointer(cqb.cq_opts(4, 0)), n=96, wsb=64), 3),
    (dict(kc=ODD), 1), (dict(vc=ODD), 1), (dict(kt=ODD), 1), (dict(ws=ODD), 1), (dict(q=ctypes.c_void_p(0x10001)), 1),
    # a code capacity below n, or one that is not a multiple of 32
    (dict(opts=ctypes.pointer(cqb.cq_opts(0, 0, 0, 32))), 1),
    (dict(opts=ctypes.pointer(cqb.cq_opts(0, 0, 0, 100))), 1),
    (dict(opts=ctypes.pointer(cqb.cq_opts(0, 0, 0, -64))), 1),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


def _decode_noalloc(**kw):
    a = dict(q=FAKE, qdt=0, kc=FAKE, ks=FAKE, km=FAKE, vc=FAKE, vs=FAKE, vm=FAKE, kt=FAKE, vt=FAKE, tdt=0,
             B=2, Hq=32, Hkv=8, n=64, T=8, d=128, bits=1, sm=0.088, calib=None, out=FAKE, odt=0, opts=None)
    a.update(kw)
    return lib.cq_decode_attn_noalloc(a["q"], a["qdt"], a["kc"], a["ks"], a["km"], a["vc"], a["vs"], a["vm"],
                                      a["kt"], a["vt"], a["tdt"], a["B"], a["Hq"], a["Hkv"], a["n"], a["T"],
                                      a["d"], a["bits"], a["sm"], a["calib"], a["out"], a["odt"], a["opts"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(out=None), 1), (dict(kc=None), 1), (dict(T=0), 1), (dict(Hq=30), 1),
    (dict(bits=5), 1), (dict(d=64), 2), (dict(kc=ODD), 1),
    (dict(opts=ctypes.pointer(cqb.cq_opts(8, 0))), 1),
    (dict(opts=ctypes.pointer(cqb.cq_opts(3, 0)), Hq=64), 2),
    # the generic schedule's scores of 64 x 32 heads x 8192 tokens take 64 MiB:
    # beyond the fixed scratch, refused before anything is enqueued
    (dict(opts=ctypes.pointer(cqb.cq_opts(1, 0)), B=64, n=8192, T=0, kt=None, vt=None), 3),
    (dict(B=0, q=None, out=None, kc=None, ks=None, km=None, vc=None, vs=None, vm=None, kt=None, vt=None), 0),
])
def test_decode_noalloc_rejects(kw, status):
    assert _decode_noalloc(**kw) == status


def test_noalloc_scratch_size_is_declared():
    text = open(os.path.join(ROOT, "include", "cq.h")).read()
    assert "#define CQ_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in text


def test_calibrate_rejects():
    c = cqb.cq_calib(1, 0.9, 0.0, 0.8, 0.0)
    assert lib.cq_calibrate(FAKE, 4, 0, ctypes.byref(c), FAKE, None, None) == 1
    assert lib.cq_calibrate(None, 4, 8, ctypes.byref(c), FAKE, None, None) == 1
    assert lib.cq_calibrate(FAKE, 4, 8, None, FAKE, None, None) == 1
    assert lib.cq_calibrate(FAKE, -1, 8, ctypes.byref(c), FAKE, None, None) == 1


def test_fp16_baseline_rejects():
    f = lib.cq_decode_attn_fp16
    assert f(None, FAKE, FAKE, 1, 32, 8, 64, 128, 0.1, FAKE, FAKE, 1 << 30, None) == 1
    assert f(FAKE, FAKE, FAKE, 1, 32, 8, 0, 128, 0.1, FAKE, FAKE, 1 << 30, None) == 1
    assert f(FAKE, FAKE, FAKE, 1, 32, 8, 64, 64, 0.1, FAKE, FAKE, 1 << 30, None) == 2
    assert f(FAKE, FAKE, FAKE, 1, 32, 8, 64, 128, 0.1, FAKE, None, 0, None) == 3
    assert f(FAKE, ODD, FAKE, 1, 32, 8, 64, 128, 0.1, FAKE, FAKE, 1 << 30, None) == 1


def test_empty_batch_is_a_no_op_without_gpu_work():
    # B == 0: valid, nothing to do, no pointer needed
    assert _quant(B=0, x=None, codes=None, scale=None, minv=None, ws=None, wsb=0) == 0
    assert _decode(B=0, q=None, out=None, kc=None, ks=None, km=None, vc=None, vs=None, vm=None, kt=None,
                   vt=None, ws=None, wsb=0) == 0


def test_binding_has_no_cpu_fallback():
    src = open(os.path.join(ROOT, "extreme_bit_kv_amd", "_binding.py")).read()
    assert "import oracle" not in src and "from oracle" not in src
    for f in os.listdir(os.path.join(ROOT, "extreme_bit_kv_amd", "csrc")):
        assert "oracle" not in open(os.path.join(ROOT, "extreme_bit_kv_amd", "csrc", f)).read()


def test_score_entry_points_reject():
    """cq_visual_scores / cq_scores_fp16 argument checks (no launch happens)."""
    sm = 0.088
    vs = lambda **kw: lib.cq_visual_scores(*[kw.get(k, v) for k, v in (
        ("q", FAKE), ("qdt", 0), ("kc", FAKE), ("ks", FAKE), ("km", FAKE), ("B", 2), ("Hq", 32), ("Hkv", 8),
        ("n", 64), ("d", 128), ("bits", 1), ("sm", sm), ("out", FAKE), ("st", None))])
    assert vs(q=None) == 1 and vs(kc=None) == 1 and vs(out=None) == 1
    assert vs(n=0) == 1 and vs(bits=3) == 1 and vs(Hq=30) == 1 and vs(qdt=2) == 1
    assert vs(kc=ODD) == 1 and vs(sm=float("nan")) == 1
    assert vs(d=64) == 2 and vs(Hq=80) == 2
    f16 = lambda **kw: lib.cq_scores_fp16(*[kw.get(k, v) for k, v in (
        ("q", FAKE), ("k", FAKE), ("B", 2), ("Hq", 32), ("Hkv", 8), ("N", 64), ("d", 128), ("sm", sm),
        ("out", FAKE), ("st", None))])
    assert f16(q=None) == 1 and f16(k=None) == 1 and f16(out=None) == 1 and f16(N=0) == 1
    assert f16(k=ODD) == 1 and f16(Hq=30) == 1
    assert f16(d=64) == 2 and f16(Hq=80) == 2


def _range(**kw):
    a = dict(x=FAKE, dt=cqb.CQ_F16, B=2, H=8, rows=1024, t0=0, m=512, d=128, mn=FAKE, mx=FAKE, reset=1, grew=None)
    a.update(kw)
    return lib.cq_kv_range_update(a["x"], a["dt"], a["B"], a["H"], a["rows"], a["t0"], a["m"], a["d"], a["mn"],
                                  a["mx"], a["reset"], a["grew"], None)


def _rows(**kw):
    a = dict(x=FAKE, dt=cqb.CQ_F16, B=2, H=8, rows=1024, t0=0, m=512, d=128, bits=1, layout=cqb.CQ_LAYOUT_K,
             mn=FAKE, mx=FAKE, mask=None, n=1024, codes=FAKE, scale=FAKE, minv=FAKE)
    a.update(kw)
    return lib.cq_quantize_kv_rows(a["x"], a["dt"], a["B"], a["H"], a["rows"], a["t0"], a["m"], a["d"], a["bits"],
                                   a["layout"], a["mn"], a["mx"], a["mask"], a["n"], a["codes"], a["scale"],
                                   a["minv"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(mn=None), 1), (dict(mx=None), 1), (dict(dt=5), 1), (dict(t0=-32), 1),
    (dict(m=-1), 1), (dict(t0=768), 1),                # t0 + m > x_rows
    (dict(m=0), 1),                                    # a reset needs a row
    (dict(reset=2), 1), (dict(B=-1), 1), (dict(x=ODD), 1), (dict(grew=ctypes.c_void_p(0x10002)), 1),
    (dict(d=64, rows=64, m=64), 2),
])
def test_range_update_rejects(kw, status):
    assert _range(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(mn=None), 1), (dict(mx=None), 1), (dict(scale=None), 1),
    (dict(minv=None), 1), (dict(bits=3), 1), (dict(layout=2), 1), (dict(dt=4), 1),
    (dict(t0=16), 1),                                  # not on a 32-token boundary
    (dict(m=100), 1),                                  # ragged, and not the segment's end
    (dict(t0=768), 1), (dict(n=512, t0=32), 1),        # past the code buffer
    (dict(rows=256), 1),                               # past x
    (dict(x=ODD), 1), (dict(codes=ODD), 1), (dict(mask=ctypes.c_void_p(0x10002)), 1),
    (dict(d=48), 1), (dict(d=64, rows=64, m=64, n=64), 2),
])
def test_quantize_rows_rejects(kw, status):
    assert _rows(**kw) == status


def test_rows_calls_without_work_are_no_ops():
    assert _range(B=0, x=None, mn=None, mx=None) == 0
    assert _range(m=0, reset=0, x=None) == 0                        # nothing to merge, no flag to clear
    assert _rows(B=0, x=None, codes=None, mn=None, mx=None, scale=None, minv=None) == 0
    assert _rows(m=0, x=None, codes=None, scale=None, minv=None) == 0


def _pair(**kw):
    a = dict(k=FAKE, v=FAKE, dt=cqb.CQ_F16, B=1, H=1, n=64, d=128, bits=1, kc=FAKE, ks=FAKE, km=FAKE, vc=FAKE,
             vs=FAKE, vm=FAKE, ws=FAKE, wsb=1 << 30, opts=None)
    a.update(kw)
    return lib.cq_quantize_kv_pair(a["k"], a["v"], a["dt"], a["B"], a["H"], a["n"], a["d"], a["bits"], a["kc"],
                                   a["ks"], a["km"], a["vc"], a["vs"], a["vm"], a["ws"], a["wsb"], a["opts"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), 1), (dict(v=None), 1), (dict(kc=None), 1), (dict(vc=None), 1), (dict(ks=None), 1),
    (dict(vm=None), 1), (dict(bits=3), 1), (dict(dt=7), 1), (dict(n=-1), 1), (dict(d=48), 1), (dict(d=64), 2),
    (dict(opts=ctypes.pointer(cqb.cq_opts(9, 0))), 1), (dict(v=ODD), 1), (dict(vc=ODD), 1), (dict(ws=ODD), 1),
    (dict(opts=ctypes.pointer(cqb.cq_opts(0, 0, -1))), 1),                # negative poll limit
])
def test_quantize_pair_rejects(kw, status):
    assert _pair(**kw) == status


def test_quantize_pair_workspace_query():
    assert lib.cq_quantize_kv_pair_workspace(64, 8, 8192, 128, 1) >= lib.cq_quantize_kv_workspace(64, 8, 8192, 128, 1)
    assert lib.cq_quantize_kv_pair_workspace(1, 1, 256, 128, 3) == 0
    assert _pair(B=0, k=None, v=None, kc=None, ks=None, km=None, vc=None, vs=None, vm=None, ws=None, wsb=0) == 0


def test_quantize_status_rejects_before_any_copy():
    """cq_quantize_status validates its workspace pointer before touching the GPU."""
    assert lib.cq_quantize_status(None, None) == 1
    assert lib.cq_quantize_status(ODD, None) == 1


def test_quantize_rejects_negative_poll_limit():
    assert _quant(opts=ctypes.pointer(cqb.cq_opts(0, 0, -5))) == 1
