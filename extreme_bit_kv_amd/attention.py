"""Decode attention over a CalibQuant visual KV cache, as a drop-in module.

The pages present CalibQuant as plug-and-play: the visual part of an MLLM's
KV cache is quantized once at prefill, and every decode step attends over the
packed codes plus the full-precision text tokens (CalibQuant abstract; QbitAI
article, "Method").  This module is that integration point, and nothing more:

* ``QuantizedVisualKV`` quantizes one layer's visual K and V at prefill
  (``cq_quantize_kv_pair``, channel-wise b-bit, packed codes + scale + minimum);
* ``CalibQuantAttention`` is the per-layer decode attention
  (``cq_decode_attn``: post-scaled scores, calibration g, softmax over visual
  and text tokens, post-scaled values), with its workspace kept across calls;
* ``GraphedDecode`` captures the decode attention of every layer of one step
  as a single HIP graph and replays it: one launch per step instead of one
  per layer, with inputs written into the graph's own buffers.

All arithmetic runs in the library's HIP kernels (libcq.so); this file only
holds tensors and issues calls.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from ._binding import cq_decode_attn, cq_quantize_kv_pair, lib


class QuantizedVisualKV:
    """One layer's visual K and V, quantized at prefill.

    k_visual, v_visual: [B, Hkv, n, d] float16 or float32 on the GPU.  The
    packed codes and the per-channel scale and minimum replace them; the
    full-precision tensors can be freed afterwards."""

    def __init__(self, k_visual: Optional[torch.Tensor], v_visual: Optional[torch.Tensor], bits: int = 1):
        self.bits = bits
        if k_visual is None and v_visual is None:                 # filled by from_codes
            return
        if k_visual.shape != v_visual.shape:
            raise ValueError(f"K {tuple(k_visual.shape)} and V {tuple(v_visual.shape)} differ")
        self.B, self.Hkv, self.n, self.d = k_visual.shape
        self.n_cap = self.n
        # each (codes, scale, min); check=True synchronizes once and raises if a
        # workgroup of the fused quantizer gave up waiting (invalid codes)
        self.k, self.v = cq_quantize_kv_pair(k_visual, v_visual, bits, check=True)

    @classmethod
    def from_codes(cls, k, v, n: int, bits: int, n_cap: int = 0) -> "QuantizedVisualKV":
        """Wrap codes made elsewhere (e.g. by a chunked prefill): k and v are
        (codes, scale, min) in the K and V layouts for n_cap tokens (0: n), of
        which the first n are the segment."""
        self = cls(None, None, bits)
        self.B, self.Hkv, self.d = k[1].shape
        self.n = n
        self.n_cap = n_cap or n
        self.k, self.v = tuple(k), tuple(v)
        return self

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (*self.k, *self.v))


class CalibQuantAttention(torch.nn.Module):
    """Decode attention of one layer over a ``QuantizedVisualKV`` and an
    optional full-precision text tail [B, Hkv, T, d] (the tokens after the
    image, not quantized).

    forward(q [B, Hq, d]) -> [B, Hq, d] in q's dtype (or ``out``'s).
    ``calib`` is (a_lo, c_lo, a_hi, c_hi): the calibrated visual scores of
    each query head span [a_lo m + c_lo, a_hi M + c_hi], m and M being the
    head's visual min and max; None leaves the scores as they are."""

    def __init__(self, sm_scale: float, calib: Optional[Sequence[float]] = None):
        super().__init__()
        self.sm_scale = float(sm_scale)
        self.calib = None if calib is None else tuple(float(c) for c in calib)
        self._ws: Optional[torch.Tensor] = None

    def _workspace(self, q: torch.Tensor, cache: QuantizedVisualKV, T: int) -> Optional[torch.Tensor]:
        nbytes = lib.cq_decode_attn_workspace(q.shape[0], q.shape[1], cache.Hkv, cache.n, T, cache.d, cache.bits)
        if nbytes == 0:
            return None
        if self._ws is None or self._ws.numel() < nbytes or self._ws.device != q.device:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        return self._ws

    def forward(self, q: torch.Tensor, cache: QuantizedVisualKV, k_tail: Optional[torch.Tensor] = None,
                v_tail: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        T = 0 if k_tail is None else k_tail.shape[2]
        return cq_decode_attn(q, *cache.k, *cache.v, k_tail, v_tail, n=cache.n, bits=cache.bits,
                              sm_scale=self.sm_scale, calib=self.calib, out=out,
                              workspace=self._workspace(q, cache, T), n_cap=cache.n_cap)


class GraphedDecode:
    """The decode attention of every layer of one step, captured once as a
    HIP graph (torch.cuda.CUDAGraph) and replayed.

    layers: per layer (attention module, cache, k_tail, v_tail); shapes are
    fixed at capture.  ``step(queries)`` copies the queries into the graph's
    buffers, replays the graph, and returns the graph's output buffers (valid
    until the next step)."""

    def __init__(self, layers: Sequence, q_like: Sequence[torch.Tensor], warmup: int = 2):
        self.layers = list(layers)
        if len(q_like) != len(self.layers):
            raise ValueError("one query tensor per layer")
        self.q: List[torch.Tensor] = [torch.empty_like(q) for q in q_like]
        for dst, src in zip(self.q, q_like):
            dst.copy_(src)
        self.out: List[torch.Tensor] = [torch.empty_like(q) for q in q_like]
        side = torch.cuda.Stream(device=self.q[0].device)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):                 # warm-up outside the capture (occupancy queries)
            for _ in range(warmup):
                self._run()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._run()

    def _run(self):
        for (attn, cache, kt, vt), q, o in zip(self.layers, self.q, self.out):
            attn(q, cache, kt, vt, out=o)

    def step(self, queries: Optional[Sequence[torch.Tensor]] = None) -> List[torch.Tensor]:
        if queries is not None:
            for dst, src in zip(self.q, queries):
                dst.copy_(src)
        self.graph.replay()
        return self.out
