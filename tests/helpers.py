"""Shared helpers of the GPU parity tests: input drawing and comparisons.

Expected values always come from the oracle; the HIP library only ever
produces the values under test.
"""
import sys

import numpy as np

import oracle
from workloads import ROLE_K, ROLE_KTAIL, ROLE_V, ROLE_VTAIL, kv_numpy, kv_torch, q_numpy, q_torch

REL_TOL = 2e-3          # relative error bound on attention outputs (inf-norm per head vector)


def note(msg):
    """Name the case on stdout before a GPU step, so a failing run names it."""
    print(f"[case] {msg}", flush=True)


def f32(v):
    return float(np.float32(v))


def calib_f32(c):
    """Calibration parameters as the library sees them (float32)."""
    return None if c is None else oracle.Calib(*(f32(v) for v in c))


def draw_inputs(B, Hq, Hkv, n, T, d=128, dtype="float16", seed=1, device="cuda", host=True):
    """Seeded K, V, q and tails.  host=True draws with NumPy and copies to the
    device (small shapes); host=False draws on the device (large shapes)."""
    import torch
    if host:
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        K = to(kv_numpy(seed, 0, ROLE_K, B, Hkv, n, d, dtype))
        V = to(kv_numpy(seed, 0, ROLE_V, B, Hkv, n, d, dtype))
        q = to(q_numpy(seed, 0, B, Hq, d, dtype))
        kt = to(kv_numpy(seed, 0, ROLE_KTAIL, B, Hkv, T, d, dtype)) if T else None
        vt = to(kv_numpy(seed, 0, ROLE_VTAIL, B, Hkv, T, d, dtype)) if T else None
    else:
        K = kv_torch(seed, 0, ROLE_K, B, Hkv, n, d, dtype, device)
        V = kv_torch(seed, 0, ROLE_V, B, Hkv, n, d, dtype, device)
        q = q_torch(seed, 0, B, Hq, d, dtype, device)
        kt = kv_torch(seed, 0, ROLE_KTAIL, B, Hkv, T, d, dtype, device) if T else None
        vt = kv_torch(seed, 0, ROLE_VTAIL, B, Hkv, T, d, dtype, device) if T else None
    return K, V, q, kt, vt


def words_u32(t):
    """int32 device words -> uint32 host array."""
    return t.cpu().numpy().view(np.uint32)


def rel_err(got, ref):
    """max over head vectors of ||got - ref||_inf / max(||ref||_inf, 1e-6)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-6)
    return float((num / den).max())


def oracle_unit_decode(q_h, K_u, V_u, kt_u, vt_u, bits, sm, calib):
    """Oracle decode of one (batch, kv head) from raw cache blocks (host arrays)."""
    kc, ks, km, _ = oracle.quantize_unit(K_u, bits)
    vc, vs, vm, _ = oracle.quantize_unit(V_u, bits)
    return oracle.decode_unit(q_h, kc, ks, km, vc, vs, vm, kt_u, vt_u, sm, calib)
