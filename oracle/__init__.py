"""CPU oracle for the CalibQuant visual-KV decode path.

TEST INFRASTRUCTURE ONLY: a plain, slow, obviously-correct reference written
from the pages.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library never does.

Parity pins live in ``tests/test_oracle_quant.py`` and
``tests/test_oracle_attn.py``.  Unpinned: the authors' own calibration
parameters and target-interval definition, their tie rule and the precision of
their stored scale (no page prints them).
"""
from .cq_oracle import (Calib, attend_dense, calibrate_rows, dense_scores, code_bit_offset, decode_attn,
                        decode_unit, decode_unit_postscaled, dequant, exact_ints, nearest_f32,
                        pack, quantize, quantize_unit, quantize_with_range, range_update, unpack,
                        visual_scores)
from .brute import decode_brute, quantize_brute, quantize_brute_range

__all__ = ["Calib", "attend_dense", "calibrate_rows", "dense_scores", "code_bit_offset", "decode_attn",
           "decode_unit", "decode_unit_postscaled", "dequant", "exact_ints", "nearest_f32",
           "pack", "quantize", "quantize_unit", "quantize_with_range", "range_update", "unpack", "visual_scores",
           "decode_brute", "quantize_brute", "quantize_brute_range"]
