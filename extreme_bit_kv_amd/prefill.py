"""Quantize-on-write of the visual cache during a chunked prefill.

A prefill that runs over an image (or appends video frames) in chunks writes
the float16 K and V of each chunk into the cache.  CalibQuant quantizes the
visual cache with a per-channel range over all the segment's tokens
([ART] = QbitAI article on CalibQuant, "Method" part 1); that range is the
merge of the chunks' ranges, so it can be gathered while the chunks are
written, and the codes of the complete segment equal the one-shot codes.

``ChunkedVisualQuantizer`` drives the two library calls for one layer:

* ``append(m)`` after m more rows of the segment are written: merges them
  into the running K and V ranges (``cq_kv_range_update``: a read of the new
  rows only, while they are likely still in the Infinity Cache);
* ``finish()``: codes of the whole segment on the final range
  (``cq_quantize_kv_rows``: one streaming read, no rendezvous), returned as a
  ``QuantizedVisualKV``.

With ``eager=True`` each ``append`` also codes the new rows on the range known
so far and codes again the earlier rows of every (batch, head) whose range
the new rows widened, so the codes are those of the segment so far after
every call, and ``current()`` decodes them in place (the code buffers are
laid out for the whole segment; the decode reads the first rows).  Ranges
keep widening while the segment is short, so this re-reads the earlier rows
often; the deferred order reads each row twice in all.  All arithmetic runs
in the library's kernels.
"""
from __future__ import annotations

import torch

from ._binding import CQ_LAYOUT_K, CQ_LAYOUT_V, cq_kv_range_update, cq_quantize_kv_rows, code_words_shape
from .attention import QuantizedVisualKV


class ChunkedVisualQuantizer:
    """k_cache, v_cache: [B, Hkv, rows, d] float16/float32 caches that the
    prefill fills; the visual segment is rows [row0, row0 + n)."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, n: int, bits: int = 1, row0: int = 0,
                 eager: bool = False):
        if k_cache.shape != v_cache.shape:
            raise ValueError(f"K {tuple(k_cache.shape)} and V {tuple(v_cache.shape)} differ")
        B, H, rows, d = k_cache.shape
        if n < 1 or row0 < 0 or row0 + n > rows:
            raise ValueError(f"segment [{row0}, {row0 + n}) does not fit {rows} rows")
        self.k_cache, self.v_cache = k_cache, v_cache
        self.n, self.bits, self.row0, self.eager = n, bits, row0, eager
        self.t = 0
        dev = k_cache.device
        f32 = dict(dtype=torch.float32, device=dev)
        self.range = {L: (torch.empty((B, H, d), **f32), torch.empty((B, H, d), **f32))
                      for L in (CQ_LAYOUT_K, CQ_LAYOUT_V)}
        self.grew = {L: torch.zeros((B, H), dtype=torch.int32, device=dev) for L in (CQ_LAYOUT_K, CQ_LAYOUT_V)}
        self.out = {L: (torch.zeros(code_words_shape(B, H, n, d, bits, L), dtype=torch.int32, device=dev),
                        torch.empty((B, H, d), **f32), torch.empty((B, H, d), **f32))
                    for L in (CQ_LAYOUT_K, CQ_LAYOUT_V)}

    def _cache(self, layout):
        return self.k_cache if layout == CQ_LAYOUT_K else self.v_cache

    def append(self, m: int) -> None:
        """Rows [row0 + t, row0 + t + m) of both caches have been written."""
        if m < 1 or self.t + m > self.n:
            raise ValueError(f"{m} rows after {self.t} overrun the {self.n}-token segment")
        if self.eager and self.t % 32:
            raise ValueError("with eager codes every chunk but the last is a multiple of 32 rows")
        t, first = self.t, self.t == 0
        for L in (CQ_LAYOUT_K, CQ_LAYOUT_V):
            mn, mx = self.range[L]
            cq_kv_range_update(self._cache(L), t, m, mn, mx, reset=first, grew=self.grew[L], row0=self.row0)
            if self.eager:
                codes, scale, minv = self.out[L]
                cq_quantize_kv_rows(self._cache(L), t, m, self.bits, L, mn, mx, self.n, codes, scale, minv,
                                    row0=self.row0)
                if t:
                    cq_quantize_kv_rows(self._cache(L), 0, t, self.bits, L, mn, mx, self.n, codes, scale, minv,
                                        unit_mask=self.grew[L], row0=self.row0)
        self.t += m

    def current(self) -> QuantizedVisualKV:
        """The segment so far (eager codes only): its t rows in code buffers
        laid out for all n, for a decode between appends."""
        if not self.eager:
            raise ValueError("the segment so far is coded only with eager=True")
        if self.t == 0:
            raise ValueError("no rows appended yet")
        if self.t != self.n and self.n % 32:
            raise ValueError(f"code buffers laid out for {self.n} tokens: a decode before the end needs a multiple "
                             "of 32")
        return QuantizedVisualKV.from_codes(self.out[CQ_LAYOUT_K], self.out[CQ_LAYOUT_V], self.t, self.bits,
                                            n_cap=self.n)

    def finish(self) -> QuantizedVisualKV:
        """The quantized segment (all n rows must have been appended)."""
        if self.t != self.n:
            raise ValueError(f"{self.t} of {self.n} rows appended")
        if not self.eager:
            for L in (CQ_LAYOUT_K, CQ_LAYOUT_V):
                mn, mx = self.range[L]
                codes, scale, minv = self.out[L]
                cq_quantize_kv_rows(self._cache(L), 0, self.n, self.bits, L, mn, mx, self.n, codes, scale, minv,
                                    row0=self.row0)
        return QuantizedVisualKV.from_codes(self.out[CQ_LAYOUT_K], self.out[CQ_LAYOUT_V], self.n, self.bits)
