"""Seeded synthetic inputs for the CalibQuant visual-KV decode path.

This module only draws random numbers and names shapes.  It holds none of the
method's arithmetic (no ranges, codes, scores or softmax), so that both the CPU
oracle and the HIP path can take their inputs from it without sharing code.

Value law (a stand-in for InternVL-2.5-8B visual K/V; the pages measure real
models on unnamed prompts, and no dataset is used here):

* per (seed, layer, kv-head, K-or-V): channel means mu_j ~ N(0, 1), channel
  standard deviations sd_j ~ U(0.5, 2), and 4 of the d channels picked without
  replacement as outliers whose values are scaled by 10;
* x[b, h, i, j] = (mu_j + sd_j * z) * mult_j with z ~ N(0, 1) iid over batch,
  token and channel; text-tail tokens follow the law of the same head;
* queries q ~ N(0, 1) iid.

Small inputs come from NumPy (``*_numpy``), large ones are drawn directly on a
device with a seeded ``torch.Generator`` (``*_torch``); a test that needs the
same tensor on both sides draws it once and copies it.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

ROLE_K, ROLE_V, ROLE_KTAIL, ROLE_VTAIL, ROLE_Q = 0, 1, 2, 3, 4
_ROLE_LAW = {ROLE_K: 0, ROLE_V: 1, ROLE_KTAIL: 0, ROLE_VTAIL: 1}

N_OUTLIERS = 4
OUTLIER_MULT = 10.0


@dataclass(frozen=True)
class Config:
    """One workload: head layout, cache length, tail length, bit width, dtype."""
    name: str
    B: int
    Hq: int
    Hkv: int
    n: int
    T: int
    d: int = 128
    bits: int = 1
    dtype: str = "float16"
    calib: Optional[Tuple[float, float, float, float]] = (0.9, 0.0, 0.8, 0.0)
    layers: int = 1
    seed: int = 1
    note: str = ""


# Workloads named in the project's benchmark plan.  Calibration parameters are
# never printed on the pages; (a_lo, c_lo, a_hi, c_hi) = (0.9, 0, 0.8, 0) maps
# each score interval [m, M] onto [0.9 m, 0.8 M].
CONFIGS = {
    "tiny": Config("tiny", B=1, Hq=1, Hkv=1, n=256, T=0, dtype="float32", seed=1,
                   note="single head, fp32, oracle-sized"),
    "internvl8b_n3328": Config("internvl8b_n3328", B=16, Hq=32, Hkv=8, n=3328, T=64, seed=2,
                               note="one InternVL-2.5-8B-shaped decode layer"),
    "long_n8192": Config("long_n8192", B=64, Hq=32, Hkv=8, n=8192, T=64, seed=3,
                         note="long visual context; prefill quantize + 1 decode step"),
    "bits_sweep_b1": Config("bits_sweep_b1", B=32, Hq=32, Hkv=8, n=3328, T=64, bits=1, seed=4),
    "bits_sweep_b2": Config("bits_sweep_b2", B=32, Hq=32, Hkv=8, n=3328, T=64, bits=2, calib=None, seed=4),
    "bits_sweep_b4": Config("bits_sweep_b4", B=32, Hq=32, Hkv=8, n=3328, T=64, bits=4, calib=None, seed=4),
    "bits_sweep_b8": Config("bits_sweep_b8", B=32, Hq=32, Hkv=8, n=3328, T=64, bits=8, calib=None, seed=4),
}


def channel_law(seed: int, layer: int, kvh: int, law: int, d: int = 128):
    """(mu, sd, mult) float64 arrays of length d for one (layer, kv-head, K|V)."""
    rng = np.random.default_rng([seed, layer, kvh, law, 11])
    mu = rng.standard_normal(d)
    sd = rng.uniform(0.5, 2.0, d)
    mult = np.ones(d)
    mult[rng.choice(d, N_OUTLIERS, replace=False)] = OUTLIER_MULT
    return mu, sd, mult


def _laws(seed, layer, H, law, d):
    mus, sds, mults = zip(*(channel_law(seed, layer, h, law, d) for h in range(H)))
    return np.stack(mus), np.stack(sds), np.stack(mults)        # [H, d]


def kv_numpy(seed: int, layer: int, role: int, B: int, H: int, n: int, d: int = 128,
             dtype: str = "float16") -> np.ndarray:
    """K, V or tail tensor [B, H, n, d] drawn on the host."""
    mu, sd, mult = _laws(seed, layer, H, _ROLE_LAW[role], d)
    rng = np.random.default_rng([seed, layer, role, 23])
    z = rng.standard_normal((B, H, n, d))
    x = (mu[None, :, None, :] + sd[None, :, None, :] * z) * mult[None, :, None, :]
    return x.astype(dtype)


def q_numpy(seed: int, layer: int, B: int, Hq: int, d: int = 128, dtype: str = "float16") -> np.ndarray:
    rng = np.random.default_rng([seed, layer, ROLE_Q, 29])
    return rng.standard_normal((B, Hq, d)).astype(dtype)


def _torch_dtype(torch, dtype):
    return {"float16": torch.float16, "float32": torch.float32}[dtype]


def kv_torch(seed: int, layer: int, role: int, B: int, H: int, n: int, d: int = 128,
             dtype: str = "float16", device="cuda"):
    """K, V or tail tensor [B, H, n, d] drawn directly on ``device``.

    Draws one kv-head at a time so that the float32 temporary stays small.
    """
    import torch
    mu, sd, mult = _laws(seed, layer, H, _ROLE_LAW[role], d)
    out = torch.empty((B, H, n, d), dtype=_torch_dtype(torch, dtype), device=device)
    g = torch.Generator(device=device)
    for h in range(H):
        g.manual_seed(((seed * 1000003 + layer) * 131 + role) * 257 + h)
        mu_t = torch.as_tensor(mu[h], dtype=torch.float32, device=device)
        sd_t = torch.as_tensor(sd[h], dtype=torch.float32, device=device)
        mu_m = torch.as_tensor(mult[h], dtype=torch.float32, device=device)
        for b0 in range(0, B, 8):
            b1 = min(B, b0 + 8)
            z = torch.randn((b1 - b0, n, d), generator=g, device=device, dtype=torch.float32)
            out[b0:b1, h] = ((mu_t + sd_t * z) * mu_m).to(out.dtype)
    return out


def q_torch(seed: int, layer: int, B: int, Hq: int, d: int = 128, dtype: str = "float16", device="cuda"):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1000003 + layer) * 131 + ROLE_Q)
    z = torch.randn((B, Hq, d), generator=g, device=device, dtype=torch.float32)
    return z.to(_torch_dtype(torch, dtype))
