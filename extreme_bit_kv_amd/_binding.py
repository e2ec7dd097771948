"""ctypes binding of libcq.so: the names and arguments of include/cq.h.

Argument marshalling only.  Each function checks the torch tensors it is given
(device, dtype, contiguity, shape), allocates outputs and workspaces that the
caller did not pass, and calls the C entry point on the current HIP stream.
Every computation runs in the library's kernels; there is no Python or CPU
fallback, and importing this module fails if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python extreme_bit_kv_amd/build.py` "
                      f"(or __graft_entry__.build()); there is no fallback path")

# PyTorch ships its own HIP runtime.  Loading torch first makes libcq bind to
# that same runtime (same soname), so one process never holds two HIP
# runtimes that disagree about the devices.
import torch  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

CQ_OK, CQ_ERR_INVALID_ARG, CQ_ERR_UNSUPPORTED, CQ_ERR_WORKSPACE, CQ_ERR_HIP, CQ_ERR_TIMEOUT = range(6)
CQ_F16, CQ_F32 = 0, 1
CQ_LAYOUT_K, CQ_LAYOUT_V = 0, 1
(CQ_PATH_AUTO, CQ_PATH_GENERIC, CQ_PATH_FAST, CQ_PATH_FAST_ONE, CQ_PATH_FAST_SPLIT, CQ_PATH_FAST_LDS, CQ_PATH_FAST_PIPE,
 CQ_PATH_FAST_WIDE) = range(8)

EXPORTED = ("cq_abi_version", "cq_last_hip_error", "cq_status_str", "cq_quantize_kv_workspace", "cq_quantize_kv",
            "cq_decode_attn_workspace", "cq_decode_attn", "cq_visual_scores", "cq_calibrate",
            "cq_decode_attn_fp16_workspace", "cq_decode_attn_fp16", "cq_scores_fp16", "cq_kv_range_update",
            "cq_quantize_kv_rows", "cq_quantize_kv_pair_workspace", "cq_quantize_kv_pair", "cq_quantize_status",
            "cq_decode_attn_noalloc")


class cq_calib(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int32), ("a_lo", ctypes.c_float), ("c_lo", ctypes.c_float),
                ("a_hi", ctypes.c_float), ("c_hi", ctypes.c_float)]


class cq_opts(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("splits", ctypes.c_int32), ("max_polls", ctypes.c_int32),
                ("n_cap", ctypes.c_int32)]


_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

lib.cq_abi_version.restype = _i32
lib.cq_abi_version.argtypes = []
lib.cq_last_hip_error.restype = _i32
lib.cq_last_hip_error.argtypes = []
lib.cq_status_str.restype = ctypes.c_char_p
lib.cq_status_str.argtypes = [_i32]
lib.cq_quantize_kv_workspace.restype = _sz
lib.cq_quantize_kv_workspace.argtypes = [_i32] * 5
lib.cq_quantize_kv.restype = _i32
lib.cq_quantize_kv.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                               ctypes.POINTER(cq_opts), _vp]
lib.cq_quantize_kv_pair_workspace.restype = _sz
lib.cq_quantize_kv_pair_workspace.argtypes = [_i32] * 5
lib.cq_quantize_kv_pair.restype = _i32
lib.cq_quantize_kv_pair.argtypes = [_vp, _vp, _i32] + [_i32] * 5 + [_vp] * 6 + [_vp, _sz, ctypes.POINTER(cq_opts), _vp]
lib.cq_quantize_status.restype = _i32
lib.cq_quantize_status.argtypes = [_vp, _vp]
lib.cq_kv_range_update.restype = _i32
lib.cq_kv_range_update.argtypes = [_vp, _i32] + [_i32] * 6 + [_vp, _vp, _i32, _vp, _vp]
lib.cq_quantize_kv_rows.restype = _i32
lib.cq_quantize_kv_rows.argtypes = [_vp, _i32] + [_i32] * 8 + [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
lib.cq_decode_attn_workspace.restype = _sz
lib.cq_decode_attn_workspace.argtypes = [_i32] * 7
lib.cq_decode_attn.restype = _i32
lib.cq_decode_attn.argtypes = ([_vp, _i32] + [_vp] * 6 + [_vp, _vp, _i32] + [_i32] * 7 +
                               [_f32, ctypes.POINTER(cq_calib), _vp, _i32, _vp, _sz,
                                ctypes.POINTER(cq_opts), _vp])
lib.cq_decode_attn_noalloc.restype = _i32
lib.cq_decode_attn_noalloc.argtypes = ([_vp, _i32] + [_vp] * 6 + [_vp, _vp, _i32] + [_i32] * 7 +
                                       [_f32, ctypes.POINTER(cq_calib), _vp, _i32, ctypes.POINTER(cq_opts), _vp])
lib.cq_visual_scores.restype = _i32
lib.cq_visual_scores.argtypes = [_vp, _i32, _vp, _vp, _vp] + [_i32] * 6 + [_f32, _vp, _vp]
lib.cq_scores_fp16.restype = _i32
lib.cq_scores_fp16.argtypes = [_vp, _vp] + [_i32] * 5 + [_f32, _vp, _vp]
lib.cq_calibrate.restype = _i32
lib.cq_calibrate.argtypes = [_vp, _i32, _i32, ctypes.POINTER(cq_calib), _vp, _vp, _vp]
lib.cq_decode_attn_fp16_workspace.restype = _sz
lib.cq_decode_attn_fp16_workspace.argtypes = [_i32] * 5
lib.cq_decode_attn_fp16.restype = _i32
lib.cq_decode_attn_fp16.argtypes = [_vp, _vp, _vp] + [_i32] * 5 + [_f32, _vp, _vp, _sz, _vp]


class CQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        extra = f" (hipError {lib.cq_last_hip_error()})" if status == CQ_ERR_HIP else ""
        super().__init__(f"{where}: {lib.cq_status_str(status).decode()}{extra}")


def _check(status: int, where: str):
    if status != CQ_OK:
        raise CQError(status, where)


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float16:
        return CQ_F16
    if t.dtype == torch.float32:
        return CQ_F32
    raise TypeError(f"expected float16 or float32, got {t.dtype}")


def _need(t, name, shape: Optional[Sequence[int]] = None, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def make_calib(calib) -> Optional[cq_calib]:
    """None / (a_lo, c_lo, a_hi, c_hi) / cq_calib -> cq_calib or None."""
    if calib is None or isinstance(calib, cq_calib):
        return calib
    a_lo, c_lo, a_hi, c_hi = calib
    return cq_calib(1, a_lo, c_lo, a_hi, c_hi)


def code_words_shape(B, H, n, d, bits, layout):
    E = 32 // bits
    return (B, H, d // E, n) if layout == CQ_LAYOUT_K else (B, H, -(-n // E), d)


def cq_quantize_status(workspace, device=None):
    """Raise CQError(CQ_ERR_TIMEOUT) if the last quantize call on `workspace`
    had a workgroup give up waiting (its outputs are then invalid).
    Synchronizes the current stream of the workspace's device."""
    _check(lib.cq_quantize_status(_ptr(workspace), _stream(device or workspace.device)), "cq_quantize_status")


def cq_quantize_kv(x, bits: int, layout: int, codes=None, scale=None, minv=None, workspace=None,
                   path: int = CQ_PATH_AUTO, check: bool = False, max_polls: int = 0):
    """x [B, H, n, d] float16/float32 -> (codes int32 words, scale f32 [B,H,d], minv f32 [B,H,d]).

    check=True synchronizes and raises CQError(CQ_ERR_TIMEOUT) if a workgroup
    gave up waiting (cq_quantize_status); max_polls is cq_opts.max_polls."""
    torch = _torch()
    _need(x, "x")
    B, H, n, d = x.shape
    dev = x.device
    if codes is None:
        codes = torch.empty(code_words_shape(B, H, n, d, bits, layout), dtype=torch.int32, device=dev)
    if scale is None:
        scale = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    if minv is None:
        minv = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _need(codes, "codes", code_words_shape(B, H, n, d, bits, layout), torch.int32, dev)
    _need(scale, "scale", (B, H, d), torch.float32, dev)
    _need(minv, "minv", (B, H, d), torch.float32, dev)
    ws_bytes = lib.cq_quantize_kv_workspace(B, H, n, d, bits)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    opts = cq_opts(path, 0, max_polls)
    st = lib.cq_quantize_kv(_ptr(x), _dtype_code(x), B, H, n, d, bits, layout, _ptr(codes), _ptr(scale),
                            _ptr(minv), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                            ctypes.byref(opts), _stream(dev))
    _check(st, "cq_quantize_kv")
    if check and workspace is not None:
        cq_quantize_status(workspace, dev)
    return codes, scale, minv


def _decode_marshal(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail, v_tail, n, bits, out,
                    out_dtype, n_cap=0):
    """Checks of the decode operands; returns (B, Hq, Hkv, T, d, tail dtype code, out, leading C args).
    The code buffers are laid out for n_cap tokens (0: n)."""
    torch = _torch()
    _need(q, "q")
    B, Hq, d = q.shape
    dev = q.device
    Hkv = k_scale.shape[1]
    T = 0 if k_tail is None else k_tail.shape[2]
    if n > 0:
        cap = n_cap or n
        _need(k_codes, "k_codes", code_words_shape(B, Hkv, cap, d, bits, CQ_LAYOUT_K), torch.int32, dev)
        _need(v_codes, "v_codes", code_words_shape(B, Hkv, cap, d, bits, CQ_LAYOUT_V), torch.int32, dev)
    for name, t in (("k_scale", k_scale), ("k_min", k_min), ("v_scale", v_scale), ("v_min", v_min)):
        _need(t, name, (B, Hkv, d), torch.float32, dev)
    tail_code = CQ_F16
    if T:
        _need(k_tail, "k_tail", (B, Hkv, T, d), None, dev)
        _need(v_tail, "v_tail", (B, Hkv, T, d), k_tail.dtype, dev)
        tail_code = _dtype_code(k_tail)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=out_dtype or q.dtype, device=dev)
    _need(out, "out", (B, Hq, d), None, dev)
    lead = (_ptr(q), _dtype_code(q), _ptr(k_codes) if n else None, _ptr(k_scale), _ptr(k_min),
            _ptr(v_codes) if n else None, _ptr(v_scale), _ptr(v_min), _ptr(k_tail) if T else None,
            _ptr(v_tail) if T else None, tail_code, B, Hq, Hkv, n, T, d, bits)
    return B, Hq, Hkv, T, d, out, lead


def cq_decode_attn(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail, v_tail, *, n: int,
                   bits: int, sm_scale: float, calib=None, out=None, out_dtype=None, workspace=None,
                   path: int = CQ_PATH_AUTO, splits: int = 0, n_cap: int = 0):
    """One decode step; q [B, Hq, d]; codes/params from cq_quantize_kv; tails [B, Hkv, T, d] or None.
    n_cap > n: the code buffers are laid out for n_cap tokens, of which the first n are attended over."""
    torch = _torch()
    B, Hq, Hkv, T, d, out, lead = _decode_marshal(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail,
                                                  v_tail, n, bits, out, out_dtype, n_cap)
    ws_bytes = lib.cq_decode_attn_workspace(B, Hq, Hkv, n, T, d, bits)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    c = make_calib(calib)
    opts = cq_opts(path, splits, 0, n_cap)
    st = lib.cq_decode_attn(*lead, float(sm_scale), None if c is None else ctypes.byref(c), _ptr(out),
                            _dtype_code(out), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                            ctypes.byref(opts), _stream(q.device))
    _check(st, "cq_decode_attn")
    return out


def cq_decode_attn_noalloc(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail, v_tail, *, n: int,
                           bits: int, sm_scale: float, out, calib=None, path: int = CQ_PATH_AUTO,
                           splits: int = 0, n_cap: int = 0):
    """cq_decode_attn into a caller's `out` with the library's fixed device
    scratch: no device memory is allocated, here or in the library."""
    _, _, _, _, _, out, lead = _decode_marshal(q, k_codes, k_scale, k_min, v_codes, v_scale, v_min, k_tail,
                                               v_tail, n, bits, out, None, n_cap)
    c = make_calib(calib)
    opts = cq_opts(path, splits, 0, n_cap)
    st = lib.cq_decode_attn_noalloc(*lead, float(sm_scale), None if c is None else ctypes.byref(c), _ptr(out),
                                    _dtype_code(out), ctypes.byref(opts), _stream(q.device))
    _check(st, "cq_decode_attn_noalloc")
    return out


def cq_visual_scores(q, k_codes, k_scale, k_min, *, n: int, bits: int, sm_scale: float, out=None):
    """Pre-softmax visual scores (before g) from packed K codes: float32 [B, Hq, n]."""
    torch = _torch()
    _need(q, "q")
    B, Hq, d = q.shape
    Hkv = k_scale.shape[1]
    _need(k_codes, "k_codes", code_words_shape(B, Hkv, n, d, bits, CQ_LAYOUT_K), torch.int32, q.device)
    for name, t in (("k_scale", k_scale), ("k_min", k_min)):
        _need(t, name, (B, Hkv, d), torch.float32, q.device)
    if out is None:
        out = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    _need(out, "out", (B, Hq, n), torch.float32, q.device)
    st = lib.cq_visual_scores(_ptr(q), _dtype_code(q), _ptr(k_codes), _ptr(k_scale), _ptr(k_min), B, Hq, Hkv, n,
                              d, bits, float(sm_scale), _ptr(out), _stream(q.device))
    _check(st, "cq_visual_scores")
    return out


def cq_scores_fp16(q, k, sm_scale: float, out=None):
    """Exact scores over an unquantized cache: q [B, Hq, d], k [B, Hkv, N, d] float16 -> float32 [B, Hq, N]."""
    torch = _torch()
    _need(q, "q", None, torch.float16)
    B, Hq, d = q.shape
    _need(k, "k", None, torch.float16, q.device)
    Hkv, N = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, N, d):
        raise ValueError(f"k has shape {tuple(k.shape)}, expected {(B, Hkv, N, d)}")
    if out is None:
        out = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _need(out, "out", (B, Hq, N), torch.float32, q.device)
    st = lib.cq_scores_fp16(_ptr(q), _ptr(k), B, Hq, Hkv, N, d, float(sm_scale), _ptr(out), _stream(q.device))
    _check(st, "cq_scores_fp16")
    return out


def cq_calibrate(scores, calib, out=None, row_minmax=None):
    """scores [R, n] float32 -> g(scores) (float32), optionally (m, M) per row."""
    torch = _torch()
    _need(scores, "scores", None, torch.float32)
    R, n = scores.shape
    if out is None:
        out = torch.empty_like(scores)
    _need(out, "out", (R, n), torch.float32, scores.device)
    if row_minmax is not None:
        _need(row_minmax, "row_minmax", (R, 2), torch.float32, scores.device)
    c = make_calib(calib) or cq_calib(0, 1.0, 0.0, 1.0, 0.0)
    st = lib.cq_calibrate(_ptr(scores), R, n, ctypes.byref(c), _ptr(out), _ptr(row_minmax),
                          _stream(scores.device))
    _check(st, "cq_calibrate")
    return out


def cq_decode_attn_fp16(q, k, v, sm_scale: float, out=None, workspace=None):
    """Unquantized baseline: q [B, Hq, d], k/v [B, Hkv, N, d], all float16."""
    torch = _torch()
    _need(q, "q", None, torch.float16)
    B, Hq, d = q.shape
    _need(k, "k", None, torch.float16, q.device)
    Hkv, N = k.shape[1], k.shape[2]
    _need(v, "v", (B, Hkv, N, d), torch.float16, q.device)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (B, Hq, d), torch.float16, q.device)
    ws_bytes = lib.cq_decode_attn_fp16_workspace(B, Hq, Hkv, N, d)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib.cq_decode_attn_fp16(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, d, float(sm_scale), _ptr(out),
                                 _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                 _stream(q.device))
    _check(st, "cq_decode_attn_fp16")
    return out


def cq_quantize_kv_pair(k, v, bits: int, k_out=None, v_out=None, workspace=None, path: int = CQ_PATH_AUTO,
                        check: bool = False, max_polls: int = 0):
    """One layer's K and V [B, H, n, d] (same shape and dtype) quantized in one
    call.  Returns ((k_codes, k_scale, k_min), (v_codes, v_scale, v_min)) in
    the K and V layouts; k_out / v_out may pass those buffers.  check and
    max_polls as for cq_quantize_kv."""
    torch = _torch()
    _need(k, "k")
    _need(v, "v", tuple(k.shape), k.dtype, k.device)
    B, H, n, d = k.shape
    dev = k.device

    def outs(given, layout, name):
        if given is None:
            given = (torch.empty(code_words_shape(B, H, n, d, bits, layout), dtype=torch.int32, device=dev),
                     torch.empty((B, H, d), dtype=torch.float32, device=dev),
                     torch.empty((B, H, d), dtype=torch.float32, device=dev))
        codes, scale, minv = given
        _need(codes, f"{name}_codes", code_words_shape(B, H, n, d, bits, layout), torch.int32, dev)
        _need(scale, f"{name}_scale", (B, H, d), torch.float32, dev)
        _need(minv, f"{name}_min", (B, H, d), torch.float32, dev)
        return given
    kc, ks, km = outs(k_out, CQ_LAYOUT_K, "k")
    vc, vs, vm = outs(v_out, CQ_LAYOUT_V, "v")
    ws_bytes = lib.cq_quantize_kv_pair_workspace(B, H, n, d, bits)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    opts = cq_opts(path, 0, max_polls)
    st = lib.cq_quantize_kv_pair(_ptr(k), _ptr(v), _dtype_code(k), B, H, n, d, bits, _ptr(kc), _ptr(ks), _ptr(km),
                                 _ptr(vc), _ptr(vs), _ptr(vm), _ptr(workspace),
                                 0 if workspace is None else workspace.numel(), ctypes.byref(opts), _stream(dev))
    _check(st, "cq_quantize_kv_pair")
    if check and workspace is not None:
        cq_quantize_status(workspace, dev)
    return (kc, ks, km), (vc, vs, vm)


def _rows_ptr(x, row0: int, t0: int, m: int):
    """Pointer to row row0 of every (b, h) of x [B, H, x_rows, d]: the segment
    starts there, the unit stride stays x_rows rows."""
    B, H, x_rows, d = x.shape
    if row0 < 0 or t0 < 0 or m < 0 or row0 + t0 + m > x_rows:
        raise ValueError(f"rows [{row0 + t0}, {row0 + t0 + m}) are not inside x's {x_rows} rows")
    return ctypes.c_void_p(x.data_ptr() + row0 * d * x.element_size())


def cq_kv_range_update(x, t0: int, m: int, mn=None, mx=None, *, reset: bool, grew=None, row0: int = 0):
    """Merge rows [row0 + t0, row0 + t0 + m) of x [B, H, x_rows, d]
    (float16/float32) into the running per-channel range mn, mx (float32
    [B, H, d], updated in place; allocated when reset and not given).  grew
    (uint32 as int32 [B, H]), if given, is set to 1 where a channel's range
    became wider.  Returns (mn, mx)."""
    torch = _torch()
    _need(x, "x")
    B, H, x_rows, d = x.shape
    dev = x.device
    xp = _rows_ptr(x, row0, t0, m)
    if mn is None or mx is None:
        if not reset:
            raise ValueError("mn and mx are required unless reset")
        mn = torch.empty((B, H, d), dtype=torch.float32, device=dev)
        mx = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _need(mn, "mn", (B, H, d), torch.float32, dev)
    _need(mx, "mx", (B, H, d), torch.float32, dev)
    if grew is not None:
        _need(grew, "grew", (B, H), torch.int32, dev)
    st = lib.cq_kv_range_update(xp, _dtype_code(x), B, H, x_rows, t0, m, d, _ptr(mn), _ptr(mx), int(reset),
                                _ptr(grew), _stream(dev))
    _check(st, "cq_kv_range_update")
    return mn, mx


def cq_quantize_kv_rows(x, t0: int, m: int, bits: int, layout: int, mn, mx, n: int, codes=None, scale=None,
                        minv=None, unit_mask=None, row0: int = 0):
    """Codes of tokens [t0, t0 + m) of the segment that starts at row row0 of
    x [B, H, x_rows, d], on the given range mn, mx (float32 [B, H, d]), into
    code words laid out for n tokens (allocated when not given).  unit_mask
    (int32 [B, H]) skips the units where it is 0.  Returns (codes, scale,
    minv)."""
    torch = _torch()
    _need(x, "x")
    B, H, x_rows, d = x.shape
    dev = x.device
    xp = _rows_ptr(x, row0, t0, m)
    shape = code_words_shape(B, H, n, d, bits, layout)
    if codes is None:
        codes = torch.zeros(shape, dtype=torch.int32, device=dev)
    if scale is None:
        scale = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    if minv is None:
        minv = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _need(codes, "codes", shape, torch.int32, dev)
    for name, t in (("mn", mn), ("mx", mx), ("scale", scale), ("minv", minv)):
        _need(t, name, (B, H, d), torch.float32, dev)
    if unit_mask is not None:
        _need(unit_mask, "unit_mask", (B, H), torch.int32, dev)
    st = lib.cq_quantize_kv_rows(xp, _dtype_code(x), B, H, x_rows, t0, m, d, bits, layout, _ptr(mn), _ptr(mx),
                                 _ptr(unit_mask), n, _ptr(codes), _ptr(scale), _ptr(minv), _stream(dev))
    _check(st, "cq_quantize_kv_rows")
    return codes, scale, minv
