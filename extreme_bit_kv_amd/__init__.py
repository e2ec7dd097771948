"""extreme_bit_kv_amd — the CalibQuant visual-KV decode path on MI355X (gfx950).

Channel-wise b-bit quantization of the visual KV cache, post-scaled decode
attention over the packed codes with the calibration map g, and an
unquantized float16 decode baseline, all as hand-written HIP kernels behind
the C ABI in include/cq.h (libcq.so).  This package is the thin Python
binding over that library; see ``_binding`` for the functions.
"""
from ._binding import (  # noqa: F401
    CQ_ERR_TIMEOUT, CQ_ERR_UNSUPPORTED, CQ_F16, CQ_F32, CQ_LAYOUT_K, CQ_LAYOUT_V, CQ_PATH_AUTO, CQ_PATH_FAST,
    CQ_PATH_FAST_LDS, CQ_PATH_FAST_ONE, CQ_PATH_FAST_PIPE, CQ_PATH_FAST_SPLIT, CQ_PATH_FAST_WIDE, CQ_PATH_GENERIC,
    EXPORTED,
    LIB_PATH, CQError, code_words_shape, cq_calib, cq_calibrate, cq_decode_attn, cq_decode_attn_fp16,
    cq_decode_attn_noalloc, cq_kv_range_update, cq_opts, cq_quantize_kv, cq_quantize_kv_pair,
    cq_quantize_kv_rows, cq_quantize_status, cq_scores_fp16, cq_visual_scores, lib, make_calib)

__all__ = [
    "CQ_ERR_TIMEOUT", "CQ_ERR_UNSUPPORTED", "CQ_F16", "CQ_F32", "CQ_LAYOUT_K", "CQ_LAYOUT_V", "CQ_PATH_AUTO",
    "CQ_PATH_FAST", "CQ_PATH_FAST_LDS", "CQ_PATH_FAST_ONE", "CQ_PATH_FAST_PIPE", "CQ_PATH_FAST_SPLIT", "CQ_PATH_FAST_WIDE",
    "CQ_PATH_GENERIC", "EXPORTED", "LIB_PATH", "CQError", "code_words_shape", "cq_calib", "cq_calibrate",
    "cq_decode_attn", "cq_decode_attn_fp16", "cq_decode_attn_noalloc", "cq_kv_range_update", "cq_opts",
    "cq_quantize_kv", "cq_quantize_kv_pair", "cq_quantize_kv_rows", "cq_quantize_status", "cq_scores_fp16",
    "cq_visual_scores", "lib", "make_calib"
]
