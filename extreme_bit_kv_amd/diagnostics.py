"""Score-distribution diagnostic: what quantization and the calibration map g
do to the pre-softmax visual scores.

QbitAI article on CalibQuant, "Method" part 3: with 1-bit keys the
dequantized values pile up at the channel extremes and distort the attention
scores; g, an affine map of each query head's score interval, is meant to move
their distribution back toward the unquantized one (the article's figure of
"Exact", "Quant" and "Quant-C" score distributions; the figure itself is not
in the text).

For each query-head row the library computes three kinds of scores on the GPU:
  exact    cq_scores_fp16 over the float16 cache,
  quant    cq_visual_scores over the b-bit codes,
  quant-c  cq_calibrate(quant) for each calibration setting,
and this module compares them on the host:
  - KL(softmax(exact) || softmax(x)) per row, over the visual tokens (the
    attention weights the decode would use with no text tail);
  - the total-variation distance between the pooled histograms of exact and
    x scores (the figure's view);
  - the mean absolute score error.

    python -m extreme_bit_kv_amd.diagnostics [--out report.md]

runs a sweep of calibration settings on seeded synthetic outlier-channel
data (the shapes of one InternVL-2.5-8B-like layer) and prints a table.
"""
from __future__ import annotations

import argparse
import json
import math
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

from ._binding import CQ_LAYOUT_K, cq_calibrate, cq_quantize_kv, cq_scores_fp16, cq_visual_scores

Calib = Tuple[float, float, float, float]      # (a_lo, c_lo, a_hi, c_hi)


# ---------------------------------------------------------------------------
# host-side statistics (float64)
# ---------------------------------------------------------------------------

def log_softmax_rows(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, np.float64)
    z = s - s.max(axis=-1, keepdims=True)
    return z - np.log(np.exp(z).sum(axis=-1, keepdims=True))


def kl_rows(s_ref: np.ndarray, s: np.ndarray) -> np.ndarray:
    """KL(softmax(s_ref) || softmax(s)) per row, in nats."""
    lp, lq = log_softmax_rows(s_ref), log_softmax_rows(s)
    return (np.exp(lp) * (lp - lq)).sum(axis=-1)


def histogram(s: np.ndarray, edges: np.ndarray) -> np.ndarray:
    """Normalized histogram of all values of s over `edges` (values outside are clipped into the end bins)."""
    h, _ = np.histogram(np.clip(np.asarray(s, np.float64).ravel(), edges[0], edges[-1]), bins=edges)
    return h / max(1, h.sum())


def tv_distance(h1: np.ndarray, h2: np.ndarray) -> float:
    """Total-variation distance between two normalized histograms."""
    return 0.5 * float(np.abs(np.asarray(h1) - np.asarray(h2)).sum())


# ---------------------------------------------------------------------------
# the diagnostic
# ---------------------------------------------------------------------------

def score_distribution(K, q, *, sm_scale: float, calibs: Sequence[Optional[Calib]], bits: int = 1,
                       bins: int = 48) -> Dict:
    """K: float16 [B, Hkv, n, d] visual keys on the device; q: float16 [B, Hq, d].

    Returns {"exact_hist", "edges", "settings": [{"calib", "kl_mean", "kl_median", "tv", "mae", "hist"}]},
    where the first setting is always the uncalibrated quantized cache (calib None)."""
    import torch
    B, Hkv, n, d = K.shape
    Hq = q.shape[1]
    exact = cq_scores_fp16(q, K, sm_scale)
    kc, ks, km = cq_quantize_kv(K, bits, CQ_LAYOUT_K)
    quant = cq_visual_scores(q, kc, ks, km, n=n, bits=bits, sm_scale=sm_scale)
    rows = quant.view(B * Hq, n)
    variants = [(None, rows)]
    for c in calibs:
        if c is not None:
            variants.append((tuple(c), cq_calibrate(rows, c)))
    torch.cuda.synchronize()
    ex = exact.view(B * Hq, n).cpu().numpy().astype(np.float64)
    lo, hi = float(ex.min()), float(ex.max())
    pad = 0.25 * (hi - lo) + 1e-6
    edges = np.linspace(lo - pad, hi + pad, bins + 1)
    h_ex = histogram(ex, edges)
    out = {"exact_hist": h_ex.tolist(), "edges": edges.tolist(), "bits": bits, "shape": [B, Hq, Hkv, n],
           "settings": []}
    for c, t in variants:
        s = t.cpu().numpy().astype(np.float64)
        kl = kl_rows(ex, s)
        h = histogram(s, edges)
        out["settings"].append({"calib": c, "kl_mean": float(kl.mean()), "kl_median": float(np.median(kl)),
                                "tv": tv_distance(h_ex, h), "mae": float(np.abs(s - ex).mean()),
                                "hist": h.tolist()})
    return out


def default_calibs() -> Iterable[Calib]:
    """The relative reading [tau_lo m, tau_hi M] swept, and two absolute targets."""
    for tl in (1.0, 0.9, 0.8):
        for th in (1.0, 0.9, 0.8, 0.7):
            if (tl, th) != (1.0, 1.0):
                yield (tl, 0.0, th, 0.0)
    yield (0.0, -4.0, 0.0, 4.0)
    yield (0.0, -2.0, 0.0, 6.0)


def _fmt_calib(c: Optional[Calib]) -> str:
    if c is None:
        return "quant (no g)"
    a_lo, c_lo, a_hi, c_hi = c
    if c_lo == 0.0 and c_hi == 0.0:
        return f"quant-c [{a_lo:g} m, {a_hi:g} M]"
    return f"quant-c [{a_lo:g} m + {c_lo:g}, {a_hi:g} M + {c_hi:g}]"


def report(res: Dict) -> str:
    B, Hq, Hkv, n = res["shape"]
    lines = [f"Score distributions: b={res['bits']}, B={B}, {Hq}q/{Hkv}kv, n={n} visual tokens per row.",
             "KL is KL(softmax(exact) || softmax(x)) over the visual tokens of each row; TV is the total-variation",
             "distance between the pooled score histograms (exact vs x); MAE the mean |x - exact| score error.", "",
             "| scores | KL mean | KL median | TV | MAE |", "|---|---|---|---|---|"]
    for st in res["settings"]:
        lines.append(f"| {_fmt_calib(st['calib'])} | {st['kl_mean']:.4g} | {st['kl_median']:.4g} | "
                     f"{st['tv']:.4f} | {st['mae']:.4g} |")
    return "\n".join(lines)


def main(argv=None):
    import torch
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from workloads import CONFIGS, ROLE_K, kv_torch, q_torch
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="internvl8b_n3328", help="synthetic workload (shapes and value recipe)")
    ap.add_argument("--batch", type=int, default=4, help="sequences drawn (the workload's batch is not needed)")
    ap.add_argument("--bits", type=int, default=1)
    ap.add_argument("--out", default=None, help="also write the table and the raw JSON here (markdown)")
    args = ap.parse_args(argv)
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    K = kv_torch(cfg.seed, 0, ROLE_K, args.batch, cfg.Hkv, cfg.n, cfg.d, cfg.dtype, dev)
    q = q_torch(cfg.seed, 0, args.batch, cfg.Hq, cfg.d, cfg.dtype, dev)
    res = score_distribution(K, q, sm_scale=1.0 / math.sqrt(cfg.d), calibs=list(default_calibs()), bits=args.bits)
    text = report(res)
    print(text)
    if args.out:
        with open(args.out, "w") as f:
            f.write("# Score-distribution diagnostic\n\nCommand: `python -m extreme_bit_kv_amd.diagnostics "
                    + " ".join(argv if argv is not None else sys.argv[1:]) + "`\n\n" + text + "\n\n```json\n"
                    + json.dumps({k: v for k, v in res.items() if k != "settings"} |
                                 {"settings": [{k: v for k, v in st.items() if k != "hist"}
                                               for st in res["settings"]]}) + "\n```\n")


if __name__ == "__main__":
    main()
