"""Throughput of the CalibQuant visual-KV path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_n8192]

One step is one pass of the whole path over one batch of the workload: the
prefill quantization of the full visual K and V caches (one cq_quantize_kv_pair
call: both tensors in one launch) followed by one calibrated decode-attention step for every sequence
(cq_decode_attn).  Inputs are seeded synthetic tensors already resident in HBM
when timing starts.  W untimed steps run first, then exactly K steps are timed
with the device synchronized on both sides and nothing recorded between the
calls; the same K steps then run again with HIP events on the launch stream
around every call, for the per-call times (timing-only events, created
without the system-scope fence that a default event's record performs).  One
JSON line is printed.

Beside the step it reports the decode alone with the Infinity Cache flushed
before each call, the float16 unquantized decode baseline over the same
tokens, the roofline of each kernel, and the CPU oracle timed on a bounded
sample of the same workload (the ``cpu_baseline`` leg; the only place this
file touches the oracle).

Sweeps (not the headline line; one JSON line per point, then a table):
    --sweeps [NAME ...]    bits: the bit-width sweep (b = 1, 2, 4, 8 and the
                           fp16 baseline at B=32, n=3328, one layer);
                           budget: the memory-budget sweep (32-layer stacks at
                           the largest batch that fits 5/10/20/30 GiB of KV
                           cache at 1 bit and at fp16, n = 3328 and 8192, one
                           full decode step over all layers);
                           graph: one 32-layer decode step issued layer by
                           layer and replayed as one captured HIP graph
                           (B=16 n=3328, B=64 n=8192);
                           stream: chunked prefill of the long-context
                           cache (range updates per 512/2048-token chunk,
                           final codes, eager codes) against the one-shot
                           quantization;
                           tail: the B=64 n=8192 decode at text-tail
                           lengths 64 .. 4096;
                           shapes: quantize and decode of the one-layer
                           workloads (B=16 n=3328 and B=64 n=8192) on their
                           own;
                           small: the b = 1 decode at B = 1 .. 32 (at most
                           one unit per CU), n = 3328 and 8192, on every
                           schedule that takes the shape.  No name: all seven

Profiling helpers (used to produce profiles/):
    --only {step,decode,copy}
                           run only the timed steps, only the decode
                           (--steps calls on the quantized cache, with
                           --path choosing the decode schedule), or only a
                           1 GiB copy kernel (the HBM-counter calibration
                           reference)
    --summarize DIR ...    turn rocprofv3 CSV output dirs into profiles/ files
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
METRIC = "1-bit KV decode-attn seq-steps/s + % HBM peak, n=8192, GQA 32q/8kv d=128"
PROFILES = os.path.join(ROOT, "profiles")


# ---------------------------------------------------------------------------
# algorithmic byte counts
# ---------------------------------------------------------------------------

class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence.

    A default event's record ends with a system-scope fence (a write-back and
    invalidation of the caches) that leaves the GPU idle for about 6 us and is
    counted in the interval it closes; this one records its timestamp without
    it.  Elapsed times are read only after a device synchronization.  The calls
    go to the HIP runtime the process already loaded (torch's)."""
    _hip = None
    FLAGS = 0x20000000                 # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as fh:
                for line in fh:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded (import torch and use the GPU first)")
            cls._hip = ctypes.CDLL(path)
        return cls._hip

    def __init__(self):
        import ctypes
        self._c = ctypes
        self.ev = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self.FLAGS)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if self._lib().hipEventRecord(self.ev, self._c.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = self._c.c_float()
        if self._lib().hipEventElapsedTime(self._c.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


class Flush:
    """Evicts the Infinity Cache before a cold measurement by reading 512 MiB
    (twice its size).  A read, not a fill: a fill leaves the cache full of
    dirty lines whose write-back then lands inside the timed kernel."""

    def __init__(self, dev):
        import torch
        self.buf = torch.zeros(128 << 20, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.sum()


def quant_bytes(cfg):
    """One cq_quantize_kv launch over one of K or V: read fp16 x, write codes and 2 fp32 vectors."""
    units = cfg.B * cfg.Hkv
    elem = 2 if cfg.dtype == "float16" else 4
    return units * (cfg.n * cfg.d * elem + cfg.n * cfg.d * cfg.bits // 8 + 2 * cfg.d * 4)


def decode_bytes(cfg):
    """One cq_decode_attn launch: K and V codes, fp16 tails, 4 fp32 parameter vectors, q and out."""
    units = cfg.B * cfg.Hkv
    G = cfg.Hq // cfg.Hkv
    per = 2 * cfg.n * cfg.d * cfg.bits // 8 + 2 * cfg.T * cfg.d * 2 + 4 * cfg.d * 4 + 2 * G * cfg.d * 2
    return units * per


def cache_bytes_per_seq(n, T, Hkv, d, bits, layers):
    """KV cache bytes one sequence holds over `layers` layers: 1-bit codes plus fp32
    scale/min plus the fp16 tail (bits > 0), or the plain fp16 cache (bits == 0)."""
    if bits == 0:
        return layers * Hkv * 2 * (n + T) * d * 2
    return layers * Hkv * (2 * n * d * bits // 8 + 2 * T * d * 2 + 4 * d * 4)


def fp16_bytes(cfg):
    units = cfg.B * cfg.Hkv
    G = cfg.Hq // cfg.Hkv
    return units * (2 * (cfg.n + cfg.T) * cfg.d * 2 + 2 * G * cfg.d * 2)


def _code_only(text):
    """Source text without comments and blank space: a comment edit leaves
    the kernel, and so the counters taken on it, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(*names):
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "extreme_bit_kv_amd", "csrc", name)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "quantize": ("quantize_fused.hip", "quantize_generic.hip", "cq_device.h", "cq_tile1.h"),
    "decode": ("decode_fast.hip", "decode_split.hip", "decode_generic.hip", "cq_device.h", "cq_mfma.h"),
}


def measured_traffic(workload, op):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    missing or taken from different kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(op)
    if not rec or rec.get("source_digest") != source_digest(*KERNEL_SOURCES[op]):
        return None
    return rec.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU oracle leg
# ---------------------------------------------------------------------------

def _oracle_unit(args):
    """One (batch, kv head) unit through the oracle: quantize + pack K and V,
    one calibrated decode.  Runs in a worker process; returns its seconds."""
    Ku, Vu, qu, ktu, vtu, bits, sm, calib = args
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    c32 = oracle.Calib(*(float(np.float32(v)) for v in calib)) if calib else None
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kc, ks, km, _ = oracle.quantize_unit(Ku, bits)
        vc, vs, vm, _ = oracle.quantize_unit(Vu, bits)
        oracle.pack(kc, bits, "K")
        oracle.pack(vc, bits, "V")
        oracle.decode_unit(qu, kc, ks, km, vc, vs, vm, ktu, vtu, sm, c32)
        return time.perf_counter() - t0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, K, V, q, kt, vt, sm, calib, budget_s):
    """Time the oracle (as it stands) on whole (batch, kv head) units of the
    same workload, one unit per task over a pool of worker processes (one
    thread each, as many as the host's CPU share allows, at most 16), until
    about budget_s seconds of CPU work are done; one sequence-step is Hkv
    units.  The rate is units over the pool's wall-clock time."""
    import multiprocessing as mp
    import numpy as np
    G = cfg.Hq // cfg.Hkv
    workers = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()))
    order = [(b, h) for b in range(cfg.B) for h in range(cfg.Hkv)]
    np.random.default_rng(0).shuffle(order)
    # one probe unit fixes the sample size: about budget_s seconds of CPU work
    def task(b, h):
        return (K[b, h].cpu().numpy(), V[b, h].cpu().numpy(), q[b, h * G:(h + 1) * G].cpu().numpy(),
                None if kt is None else kt[b, h].cpu().numpy(), None if vt is None else vt[b, h].cpu().numpy(),
                cfg.bits, sm, calib)
    _oracle_unit(task(*order[0]))                  # first call: imports and caches
    probe = _oracle_unit(task(*order[0]))
    units = int(min(len(order) - 1, max(workers, round(budget_s / max(probe, 1e-3)))))
    units = max(workers, units - units % workers)
    tasks = [task(b, h) for b, h in order[1:1 + units]]
    ctx = mp.get_context("spawn")                  # the parent holds a GPU context: never fork it
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_unit, tasks[:workers])    # workers started and warm before the clock
        t0 = time.perf_counter()
        cpu = sum(pool.map(_oracle_unit, tasks, chunksize=1))
        wall = time.perf_counter() - t0
    seq_steps = len(tasks) / cfg.Hkv
    return {"value": seq_steps / wall, "unit": "seq-steps/s", "cores": workers, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"{len(tasks)} (batch, kv-head) units of {cfg.name} (n={cfg.n}, d={cfg.d}, fp16): quantize + "
                      f"pack K and V and one {G}-head calibrated decode each; {workers} worker processes of one "
                      f"thread, {wall:.1f} s wall, {cpu:.1f} s of CPU work; {cfg.Hkv} units = 1 sequence-step"}


# ---------------------------------------------------------------------------
# GPU measurement
# ---------------------------------------------------------------------------

def run(args):
    import numpy as np
    import torch

    import extreme_bit_kv_amd as cqb
    from workloads import (CONFIGS, ROLE_K, ROLE_KTAIL, ROLE_V, ROLE_VTAIL, kv_torch, q_torch)

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    print(f"[bench] workload {cfg.name}: B={cfg.B} Hq={cfg.Hq} Hkv={cfg.Hkv} n={cfg.n} T={cfg.T} "
          f"bits={cfg.bits}", file=sys.stderr, flush=True)

    if args.only == "copy":
        src = torch.empty(1 << 29, dtype=torch.float16, device=dev).normal_()
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2,
                          "launches": 3}))
        return

    K = kv_torch(cfg.seed, 0, ROLE_K, cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.dtype, dev)
    V = kv_torch(cfg.seed, 0, ROLE_V, cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.dtype, dev)
    kt = kv_torch(cfg.seed, 0, ROLE_KTAIL, cfg.B, cfg.Hkv, cfg.T, cfg.d, cfg.dtype, dev) if cfg.T else None
    vt = kv_torch(cfg.seed, 0, ROLE_VTAIL, cfg.B, cfg.Hkv, cfg.T, cfg.d, cfg.dtype, dev) if cfg.T else None
    q = q_torch(cfg.seed, 0, cfg.B, cfg.Hq, cfg.d, cfg.dtype, dev)
    sm = 1.0 / float(np.sqrt(cfg.d))
    calib = cfg.calib

    # preallocated outputs and workspaces: the timed loop allocates nothing
    (kc, ks, km), (vc, vs, vm) = cqb.cq_quantize_kv_pair(K, V, cfg.bits)
    qws = torch.zeros(max(256, cqb.lib.cq_quantize_kv_pair_workspace(cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.bits)),
                      dtype=torch.uint8, device=dev)
    dws = torch.empty(max(1, cqb.lib.cq_decode_attn_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.n, cfg.T, cfg.d,
                                                              cfg.bits)), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.float16, device=dev)

    def quant():
        cqb.cq_quantize_kv_pair(K, V, cfg.bits, k_out=(kc, ks, km), v_out=(vc, vs, vm), workspace=qws)

    def decode(path=cqb.CQ_PATH_AUTO):
        cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=cfg.n, bits=cfg.bits, sm_scale=sm,
                           calib=calib, out=out, workspace=dws, path=path)

    if args.only == "decode":
        path = getattr(cqb, "CQ_PATH_" + args.path.upper())
        ev = [TimingEvent() for _ in range(args.steps + 1)]
        for _ in range(args.warmup):
            decode(path)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for k in range(args.steps):
            decode(path)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        ts = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
        print(json.dumps({"workload": cfg.name, "path": args.path, "calls": args.steps,
                          "decode_ms_median": float(np.median(ts))}), flush=True)
        return

    for _ in range(args.warmup):
        quant()
        decode()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # the timed steps: nothing between the calls (an event recorded on the
    # stream costs about 6 us of idle GPU, its release fence, so a step
    # timed call by call would carry that twice)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        quant()
        decode()
    t_enq = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    print(f"[bench] host enqueue {(t_enq - t0) * 1e3 / args.steps:.3f} ms/step", file=sys.stderr, flush=True)
    # the same steps again, with events at step boundaries and between the two
    # calls, for the split into calls (a step's decode ends at the event where
    # the next step's quantize starts, so every step carries two events)
    ev = [TimingEvent() for _ in range(2 * args.steps + 1)]
    ev[0].record(stream)
    for k in range(args.steps):
        quant()
        ev[2 * k + 1].record(stream)
        decode()
        ev[2 * k + 2].record(stream)
    torch.cuda.synchronize()
    # every quantize call completed its waits (else its codes would be
    # invalid): the last call's status word, and the header word that any
    # timed-out call since the workspace was zeroed sets
    cqb.cq_quantize_status(qws)
    if int(qws[4:8].view(torch.int32).item()) != 0:
        raise RuntimeError("a quantize call of the run timed out waiting; its codes were invalid")
    tq_all = np.array([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]) * 1e-3
    td_all = np.array([ev[2 * k + 1].elapsed_time(ev[2 * k + 2]) for k in range(args.steps)]) * 1e-3
    tq, td = float(np.mean(tq_all)), float(np.mean(td_all))
    print(f"[bench] timed {args.steps} steps: {wall * 1e3 / args.steps:.3f} ms/step", file=sys.stderr, flush=True)
    if args.only == "step":
        print(json.dumps({"workload": cfg.name, "steps": args.steps, "ms_per_step": wall * 1e3 / args.steps,
                          "per_call_ms": {"quantize_kv_pair": tq * 1e3, "decode_in_step": td * 1e3}}), flush=True)
        return

    # decode alone with the Infinity Cache flushed before every call
    scratch = Flush(dev)
    cold = []
    for _ in range(max(50, args.steps)):
        scratch()
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        decode()
        b.record(stream)
        cold.append((a, b))
    torch.cuda.synchronize()
    tc_all = np.array([a.elapsed_time(b) for a, b in cold]) * 1e-3
    td_cold = float(np.median(tc_all))

    # float16 unquantized baseline over the same n + T tokens, same flush
    Kf = torch.cat([K, kt], dim=2) if kt is not None else K
    Vf = torch.cat([V, vt], dim=2) if vt is not None else V
    of = torch.empty_like(out)
    fws = torch.empty(max(1, cqb.lib.cq_decode_attn_fp16_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.n + cfg.T, cfg.d)),
                      dtype=torch.uint8, device=dev)
    fcold = []
    for _ in range(max(50, args.steps)):
        scratch()
        a, b = TimingEvent(), TimingEvent()
        a.record(stream)
        cqb.cq_decode_attn_fp16(q, Kf, Vf, sm, out=of, workspace=fws)
        b.record(stream)
        fcold.append((a, b))
    torch.cuda.synchronize()
    tf16 = np.median([a.elapsed_time(b) for a, b in fcold]) * 1e-3
    del Kf, Vf

    qb, db, fb = 2 * quant_bytes(cfg), decode_bytes(cfg), fp16_bytes(cfg)     # qb: K and V in one launch

    def roof(nbytes, secs, op):
        ach = nbytes / secs / 1e9
        traffic = measured_traffic(cfg.name, op)
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}

    def pct(a):
        return [round(float(np.percentile(a, p)) * 1e3, 4) for p in (10, 50, 90)]

    dominant = "quantize" if tq >= td else "decode"
    line = {
        "metric": METRIC,
        "value": round(cfg.B * args.steps / wall, 1),
        "unit": "seq-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in; 1-bit codes; int/f32 accumulate",
        "data": "synthetic (seeded outlier-channel K/V, N(0,1) q)",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "n": cfg.n, "T": cfg.T,
                   "d": cfg.d, "bits": cfg.bits, "calib": list(calib) if calib else None,
                   "step": "quantize K and V of the full prefill cache (one cq_quantize_kv_pair call) "
                           "+ 1 decode step"},
        "roofline": roof(qb if dominant == "quantize" else db, tq if dominant == "quantize" else td, dominant),
        "dominant_kernel": "cq_quantize_kv_pair" if dominant == "quantize" else "cq_decode_attn",
        "per_call_ms": {"quantize_kv_pair": round(tq * 1e3, 4), "decode_in_step": round(td * 1e3, 4),
                        "decode_cold": round(td_cold * 1e3, 4)},
        "per_call_ms_p10_p50_p90": {"quantize_kv_pair": pct(tq_all), "decode_in_step": pct(td_all),
                                    "decode_cold": pct(tc_all), "decode_cold_calls": len(tc_all)},
        "decode": {"seq_steps_per_s_cold": round(cfg.B / td_cold, 1),
                   "roofline_cold": roof(db, td_cold, "decode"),
                   "roofline_in_step": roof(db, td, "decode")},
        "quantize": {"roofline": roof(qb, tq, "quantize")},
        "fp16_baseline": {"kernel": "cq_decode_attn_fp16", "ms_cold": round(tf16 * 1e3, 4),
                          "seq_steps_per_s": round(cfg.B / tf16, 1),
                          "achieved_GBs": round(fb / tf16 / 1e9, 1),
                          "speedup_1bit_decode_vs_fp16": round(tf16 / td_cold, 2)},
        "bytes": {"quantize_per_launch": qb, "decode_per_launch": db, "fp16_decode_per_launch": fb},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, K, V, q, kt, vt, sm, calib, args.cpu_seconds)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# sweeps: bit widths (one layer) and KV-memory budgets (32-layer stacks)
# ---------------------------------------------------------------------------

def sweeps(args):
    import numpy as np
    import torch

    import extreme_bit_kv_amd as cqb
    from workloads import CONFIGS, ROLE_K, ROLE_KTAIL, ROLE_V, ROLE_VTAIL, Config, kv_torch, q_torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sm = 1.0 / float(np.sqrt(128.0))
    rows = []

    def note(msg):
        print(f"[sweeps] {msg}", file=sys.stderr, flush=True)

    def timed(fn, reps, flush=None):
        ts = []
        for _ in range(3):
            fn()
        for _ in range(reps):
            if flush is not None:
                flush()
            a, b = TimingEvent(), TimingEvent()
            a.record(torch.cuda.current_stream())
            fn()
            b.record(torch.cuda.current_stream())
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e-3

    def emit(row):
        rows.append(row)
        print(json.dumps(row), flush=True)

    which = set(args.sweeps) or {"bits", "budget", "graph", "stream", "tail", "shapes", "small"}
    layers, Hq, Hkv, d, T = 32, 32, 8, 128, 64
    calib = (0.9, 0.0, 0.8, 0.0)

    def bit_sweep():
        """one layer, B=32, n=3328, decode with the Infinity Cache flushed"""
        scratch = Flush(dev)
        base = CONFIGS["bits_sweep_b1"]
        K = kv_torch(base.seed, 0, ROLE_K, base.B, base.Hkv, base.n, base.d, base.dtype, dev)
        V = kv_torch(base.seed, 0, ROLE_V, base.B, base.Hkv, base.n, base.d, base.dtype, dev)
        kt = kv_torch(base.seed, 0, ROLE_KTAIL, base.B, base.Hkv, base.T, base.d, base.dtype, dev)
        vt = kv_torch(base.seed, 0, ROLE_VTAIL, base.B, base.Hkv, base.T, base.d, base.dtype, dev)
        q = q_torch(base.seed, 0, base.B, base.Hq, base.d, base.dtype, dev)
        out = torch.empty((base.B, base.Hq, base.d), dtype=torch.float16, device=dev)
        for bits in (1, 2, 4, 8):
            cfg = CONFIGS[f"bits_sweep_b{bits}"]
            note(f"bit sweep b={bits}")
            kc, ks, km = cqb.cq_quantize_kv(K, bits, cqb.CQ_LAYOUT_K)
            vc, vs, vm = cqb.cq_quantize_kv(V, bits, cqb.CQ_LAYOUT_V)
            ws = torch.empty(max(1, cqb.lib.cq_decode_attn_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.n, cfg.T, cfg.d, bits)),
                             dtype=torch.uint8, device=dev)
            t = timed(lambda: cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=cfg.n, bits=bits, sm_scale=sm,
                                                 calib=cfg.calib, out=out, workspace=ws), args.steps, scratch)
            nb = decode_bytes(cfg)
            emit({"sweep": "bits", "bits": bits, "B": cfg.B, "n": cfg.n, "T": cfg.T, "calib": cfg.calib is not None,
                  "decode_ms": round(t * 1e3, 4), "seq_steps_per_s": round(cfg.B / t, 1),
                  "GBs": round(nb / t / 1e9, 1), "frac_8TBs": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)})
            del kc, ks, km, vc, vs, vm, ws
        Kf, Vf = torch.cat([K, kt], dim=2), torch.cat([V, vt], dim=2)
        fws = torch.empty(max(1, cqb.lib.cq_decode_attn_fp16_workspace(base.B, base.Hq, base.Hkv, base.n + base.T,
                                                                       base.d)), dtype=torch.uint8, device=dev)
        note("bit sweep fp16 baseline")
        t = timed(lambda: cqb.cq_decode_attn_fp16(q, Kf, Vf, sm, out=out, workspace=fws), args.steps, scratch)
        nb = fp16_bytes(base)
        emit({"sweep": "bits", "bits": 16, "B": base.B, "n": base.n, "T": base.T, "calib": False,
              "decode_ms": round(t * 1e3, 4), "seq_steps_per_s": round(base.B / t, 1),
              "GBs": round(nb / t / 1e9, 1), "frac_8TBs": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)})
        del K, V, kt, vt, q, out, Kf, Vf, fws, scratch
        torch.cuda.empty_cache()

    def small_sweep():
        """b = 1 decode at one unit per CU or fewer (B = 1 .. 32, 32q/8kv, T = 64,
        n = 3328 and 8192), every schedule that takes the shape, with the
        Infinity Cache flushed before each call"""
        scratch = Flush(dev)
        paths = {"auto": cqb.CQ_PATH_AUTO, "one": cqb.CQ_PATH_FAST_ONE, "lds": cqb.CQ_PATH_FAST_LDS,
                 "wide": cqb.CQ_PATH_FAST_WIDE, "pipe": cqb.CQ_PATH_FAST_PIPE, "split": cqb.CQ_PATH_FAST_SPLIT}
        for n in (3328, 8192):
            Bmax = 32
            K = kv_torch(7, 0, ROLE_K, Bmax, Hkv, n, d, "float16", dev)
            V = kv_torch(7, 0, ROLE_V, Bmax, Hkv, n, d, "float16", dev)
            kc_all, ks_all, km_all = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
            vc_all, vs_all, vm_all = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
            del K, V
            kt_all = kv_torch(7, 0, ROLE_KTAIL, Bmax, Hkv, T, d, "float16", dev)
            vt_all = kv_torch(7, 0, ROLE_VTAIL, Bmax, Hkv, T, d, "float16", dev)
            q_all = q_torch(7, 0, Bmax, Hq, d, "float16", dev)
            for B in (1, 2, 4, 8, 16, 32):
                cfg = Config(f"small_B{B}_n{n}", B=B, Hq=Hq, Hkv=Hkv, n=n, T=T, seed=7)
                kc, ks, km, vc, vs, vm, kt, vt, q = (x[:B] for x in (kc_all, ks_all, km_all, vc_all, vs_all, vm_all,
                                                                      kt_all, vt_all, q_all))
                out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
                ws = torch.empty(max(1, cqb.lib.cq_decode_attn_workspace(B, Hq, Hkv, n, T, d, 1)),
                                 dtype=torch.uint8, device=dev)
                row = {"sweep": "small", "B": B, "n": n, "T": T}
                for name, path in paths.items():
                    note(f"small B={B} n={n} {name}")
                    try:
                        t = timed(lambda: cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=1,
                                                             sm_scale=sm, calib=calib, out=out, workspace=ws,
                                                             path=path), args.steps, scratch)
                    except cqb.CQError:
                        continue                       # the schedule does not take the shape
                    row[name + "_us"] = round(t * 1e6, 2)
                nb = decode_bytes(cfg)
                best = min(v for k, v in row.items() if k.endswith("_us"))
                row["auto_frac_8TBs"] = round(nb / (row["auto_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                row["best_us"] = best
                emit(row)
            del kc_all, ks_all, km_all, vc_all, vs_all, vm_all, kt_all, vt_all, q_all
            torch.cuda.empty_cache()
        del scratch

    def tail_sweep():
        """B=64, n=8192, one layer, decode with the Infinity Cache flushed at
        text-tail lengths on both sides of the fused pass's 256 tokens"""
        scratch = Flush(dev)
        base = CONFIGS["long_n8192"]
        K = kv_torch(base.seed, 0, ROLE_K, base.B, base.Hkv, base.n, base.d, base.dtype, dev)
        V = kv_torch(base.seed, 0, ROLE_V, base.B, base.Hkv, base.n, base.d, base.dtype, dev)
        q = q_torch(base.seed, 0, base.B, base.Hq, base.d, base.dtype, dev)
        kc, ks, km = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
        vc, vs, vm = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
        del K, V
        out = torch.empty((base.B, base.Hq, base.d), dtype=torch.float16, device=dev)
        for T_ in (64, 256, 257, 1024, 4096):
            cfg = Config(f"long_n8192_T{T_}", B=base.B, Hq=base.Hq, Hkv=base.Hkv, n=base.n, T=T_, seed=base.seed)
            note(f"tail sweep T={T_}")
            kt = kv_torch(base.seed, 0, ROLE_KTAIL, base.B, base.Hkv, T_, base.d, base.dtype, dev)
            vt = kv_torch(base.seed, 0, ROLE_VTAIL, base.B, base.Hkv, T_, base.d, base.dtype, dev)
            ws = torch.empty(max(1, cqb.lib.cq_decode_attn_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.n, T_, cfg.d, 1)),
                             dtype=torch.uint8, device=dev)
            t = timed(lambda: cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=cfg.n, bits=1, sm_scale=sm,
                                                 calib=cfg.calib, out=out, workspace=ws), args.steps, scratch)
            nb = decode_bytes(cfg)
            emit({"sweep": "tail", "B": cfg.B, "n": cfg.n, "T": T_, "decode_ms": round(t * 1e3, 4),
                  "seq_steps_per_s": round(cfg.B / t, 1), "GBs": round(nb / t / 1e9, 1),
                  "frac_8TBs": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)})
            del kt, vt, ws
        del kc, ks, km, vc, vs, vm, q, out, scratch
        torch.cuda.empty_cache()

    def shapes_sweep():
        """the single-layer workloads on their own: quantize of K and V, and one
        decode with the Infinity Cache flushed"""
        scratch = Flush(dev)
        for name in ("internvl8b_n3328", "long_n8192"):
            cfg = CONFIGS[name]
            note(f"shapes {name}")
            K = kv_torch(cfg.seed, 0, ROLE_K, cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.dtype, dev)
            V = kv_torch(cfg.seed, 0, ROLE_V, cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.dtype, dev)
            kt = kv_torch(cfg.seed, 0, ROLE_KTAIL, cfg.B, cfg.Hkv, cfg.T, cfg.d, cfg.dtype, dev)
            vt = kv_torch(cfg.seed, 0, ROLE_VTAIL, cfg.B, cfg.Hkv, cfg.T, cfg.d, cfg.dtype, dev)
            q = q_torch(cfg.seed, 0, cfg.B, cfg.Hq, cfg.d, cfg.dtype, dev)
            kw = cqb.code_words_shape(cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.bits, cqb.CQ_LAYOUT_K)
            vw = cqb.code_words_shape(cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.bits, cqb.CQ_LAYOUT_V)
            f32 = dict(dtype=torch.float32, device=dev)
            kc, vc = torch.empty(kw, dtype=torch.int32, device=dev), torch.empty(vw, dtype=torch.int32, device=dev)
            ks, km, vs, vm = (torch.empty((cfg.B, cfg.Hkv, cfg.d), **f32) for _ in range(4))
            qws = torch.zeros(max(256, cqb.lib.cq_quantize_kv_pair_workspace(cfg.B, cfg.Hkv, cfg.n, cfg.d, cfg.bits)),
                              dtype=torch.uint8, device=dev)
            tq = timed(lambda: cqb.cq_quantize_kv_pair(K, V, cfg.bits, k_out=(kc, ks, km), v_out=(vc, vs, vm),
                                                       workspace=qws), args.steps, scratch)
            cqb.cq_quantize_status(qws)
            out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.float16, device=dev)
            ws = torch.empty(max(1, cqb.lib.cq_decode_attn_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.n, cfg.T, cfg.d,
                                                                     cfg.bits)), dtype=torch.uint8, device=dev)
            td = timed(lambda: cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=cfg.n, bits=cfg.bits,
                                                  sm_scale=sm, calib=cfg.calib, out=out, workspace=ws),
                       args.steps, scratch)
            qb, db = 2 * quant_bytes(cfg), decode_bytes(cfg)
            emit({"sweep": "shapes", "workload": name, "B": cfg.B, "n": cfg.n, "T": cfg.T,
                  "quantize_ms": round(tq * 1e3, 4), "quantize_GBs": round(qb / tq / 1e9, 1),
                  "quantize_frac_8TBs": round(qb / tq / 1e9 / HBM_PEAK_GBS, 4),
                  "decode_ms": round(td * 1e3, 4), "decode_seq_steps_per_s": round(cfg.B / td, 1),
                  "decode_GBs": round(db / td / 1e9, 1), "decode_frac_8TBs": round(db / td / 1e9 / HBM_PEAK_GBS, 4)})
            del K, V, kt, vt, q, kc, vc, ks, km, vs, vm, qws, out, ws
            torch.cuda.empty_cache()
        del scratch

    def budget_sweep():
        """32 layers, the largest batch whose cache fits the budget"""
        for n in (3328, 8192):
            for gib in (5, 10, 20, 30):
                budget = gib << 30
                for bits in (1, 0):
                    per_seq = cache_bytes_per_seq(n, T, Hkv, d, bits, layers)
                    B = budget // per_seq
                    note(f"budget {gib} GiB n={n} {'1-bit' if bits else 'fp16'}: batch {B}, building {layers} layers")
                    cache = []
                    for layer in range(layers):
                        seed = 5
                        K = kv_torch(seed, layer, ROLE_K, B, Hkv, n, d, "float16", dev)
                        V = kv_torch(seed, layer, ROLE_V, B, Hkv, n, d, "float16", dev)
                        kt = kv_torch(seed, layer, ROLE_KTAIL, B, Hkv, T, d, "float16", dev)
                        vt = kv_torch(seed, layer, ROLE_VTAIL, B, Hkv, T, d, "float16", dev)
                        q = q_torch(seed, layer, B, Hq, d, "float16", dev)
                        if bits:
                            kc = cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K)
                            vc = cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)
                            cache.append((q, kc, vc, kt, vt))
                        else:
                            cache.append((q, torch.cat([K, kt], dim=2), torch.cat([V, vt], dim=2)))
                        del K, V
                    out = torch.empty((B, Hq, d), dtype=torch.float16, device=dev)
                    if bits:
                        ws = torch.empty(max(1, cqb.lib.cq_decode_attn_workspace(B, Hq, Hkv, n, T, d, 1)),
                                         dtype=torch.uint8, device=dev)

                        def step():
                            for (q, (kc, ks, km), (vc, vs, vm), kt, vt) in cache:
                                cqb.cq_decode_attn(q, kc, ks, km, vc, vs, vm, kt, vt, n=n, bits=1, sm_scale=sm,
                                                   calib=calib, out=out, workspace=ws)
                        nb = layers * B * Hkv * (2 * n * d // 8 + 2 * T * d * 2 + 4 * d * 4 + 2 * (Hq // Hkv) * d * 2)
                    else:
                        ws = torch.empty(max(1, cqb.lib.cq_decode_attn_fp16_workspace(B, Hq, Hkv, n + T, d)),
                                         dtype=torch.uint8, device=dev)

                        def step():
                            for (q, Kf, Vf) in cache:
                                cqb.cq_decode_attn_fp16(q, Kf, Vf, sm, out=out, workspace=ws)
                        nb = layers * B * Hkv * (2 * (n + T) * d * 2 + 2 * (Hq // Hkv) * d * 2)
                    t = timed(step, max(3, args.steps // 4))
                    emit({"sweep": "budget", "budget_GiB": gib, "n": n, "T": T, "layers": layers,
                          "cache": "1-bit" if bits else "fp16", "B": int(B), "step_ms": round(t * 1e3, 4),
                          "seq_steps_per_s": round(B / t, 1), "GBs": round(nb / t / 1e9, 1),
                          "frac_8TBs": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)})
                    del cache, out, ws
                    torch.cuda.empty_cache()

    def graph_sweep():
        """a 32-layer decode step, eager (one call per layer) and as one replayed HIP graph"""
        from extreme_bit_kv_amd.attention import CalibQuantAttention, GraphedDecode, QuantizedVisualKV
        for B, n in ((16, 3328), (64, 8192)):
            note(f"graph: 32 layers B={B} n={n}")
            attn = CalibQuantAttention(sm, calib)
            stack, qs = [], []
            for layer in range(layers):
                K = kv_torch(6, layer, ROLE_K, B, Hkv, n, d, "float16", dev)
                V = kv_torch(6, layer, ROLE_V, B, Hkv, n, d, "float16", dev)
                stack.append((attn, QuantizedVisualKV(K, V, bits=1),
                              kv_torch(6, layer, ROLE_KTAIL, B, Hkv, T, d, "float16", dev),
                              kv_torch(6, layer, ROLE_VTAIL, B, Hkv, T, d, "float16", dev)))
                qs.append(q_torch(6, layer, B, Hq, d, "float16", dev))
                del K, V
            outs = [torch.empty_like(q) for q in qs]

            def eager():
                for (a, c, kt, vt), q, o in zip(stack, qs, outs):
                    a(q, c, kt, vt, out=o)
            graphed = GraphedDecode(stack, qs)
            te = timed(eager, args.steps)
            tg = timed(graphed.step, args.steps)
            nb = layers * B * Hkv * (2 * n * d // 8 + 2 * T * d * 2 + 4 * d * 4 + 2 * (Hq // Hkv) * d * 2)
            for mode, t in (("eager", te), ("graph", tg)):
                emit({"sweep": "graph", "mode": mode, "n": n, "T": T, "layers": layers, "B": B,
                      "step_ms": round(t * 1e3, 4), "seq_steps_per_s": round(B / t, 1), "GBs": round(nb / t / 1e9, 1),
                      "frac_8TBs": round(nb / t / 1e9 / HBM_PEAK_GBS, 4)})
            del stack, qs, outs, graphed
            torch.cuda.empty_cache()

    def stream_sweep():
        """chunked prefill of the long-context cache (B=64, 8 kv heads, n=8192):
        per-chunk range updates and the final row codes, deferred and eager,
        against the one-shot fused quantization"""
        from extreme_bit_kv_amd.prefill import ChunkedVisualQuantizer
        B, H, n = 64, 8, 8192
        K = kv_torch(7, 0, ROLE_K, B, H, n, d, "float16", dev)
        V = kv_torch(7, 0, ROLE_V, B, H, n, d, "float16", dev)
        x_bytes = B * H * n * d * 2
        code_bytes = B * H * n * d // 8
        t = timed(lambda: (cqb.cq_quantize_kv(K, 1, cqb.CQ_LAYOUT_K), cqb.cq_quantize_kv(V, 1, cqb.CQ_LAYOUT_V)),
                  args.steps)
        emit({"sweep": "stream", "mode": "one-shot", "chunk": n, "B": B, "n": n, "ms": round(t * 1e3, 4),
              "seq_steps_per_s": round(B / t, 1), "GBs": round(2 * (x_bytes + code_bytes) / t / 1e9, 1),
              "frac_8TBs": round(2 * (x_bytes + code_bytes) / t / 1e9 / HBM_PEAK_GBS, 4)})
        for chunk in (512, 2048):
            note(f"stream: chunk {chunk}")
            q = ChunkedVisualQuantizer(K, V, n, bits=1)

            def gather():
                q.t = 0
                for _ in range(n // chunk):
                    q.append(chunk)
            tr = timed(gather, args.steps)
            tf = timed(q.finish, args.steps)
            for mode, tt, nb in (("range updates", tr, 2 * x_bytes), ("final codes", tf, 2 * (x_bytes + code_bytes))):
                emit({"sweep": "stream", "mode": mode, "chunk": chunk, "B": B, "n": n, "ms": round(tt * 1e3, 4),
                      "seq_steps_per_s": round(B / tt, 1), "GBs": round(nb / tt / 1e9, 1),
                      "frac_8TBs": round(nb / tt / 1e9 / HBM_PEAK_GBS, 4)})
            qe = ChunkedVisualQuantizer(K, V, n, bits=1, eager=True)

            def eager():
                qe.t = 0
                for _ in range(n // chunk):
                    qe.append(chunk)
            te = timed(eager, max(3, args.steps // 4))
            emit({"sweep": "stream", "mode": "eager", "chunk": chunk, "B": B, "n": n, "ms": round(te * 1e3, 4),
                  "seq_steps_per_s": round(B / te, 1), "GBs": None, "frac_8TBs": None})
            del q, qe
        del K, V
        torch.cuda.empty_cache()

    if "bits" in which:
        bit_sweep()
    if "budget" in which:
        budget_sweep()
    if "graph" in which:
        graph_sweep()
    if "tail" in which:
        tail_sweep()
    if "shapes" in which:
        shapes_sweep()
    if "small" in which:
        small_sweep()
    if "stream" in which:
        stream_sweep()

    # table
    print("\n| sweep | point | B | ms | seq-steps/s | GB/s | of 8 TB/s |", file=sys.stderr)
    print("|---|---|---|---|---|---|---|", file=sys.stderr)
    for r in rows:
        if r["sweep"] == "bits":
            pt, ms = (f"b={r['bits']}" if r["bits"] < 16 else "fp16") + f", n={r['n']}", r["decode_ms"]
        elif r["sweep"] == "graph":
            pt, ms = f"{r['layers']} layers, n={r['n']}, {r['mode']}", r["step_ms"]
        elif r["sweep"] == "stream":
            pt, ms = f"{r['mode']}, chunk {r['chunk']}, n={r['n']}", r["ms"]
        elif r["sweep"] == "tail":
            pt, ms = f"T={r['T']}, n={r['n']}", r["decode_ms"]
        elif r["sweep"] == "small":
            paths = ", ".join(f"{k[:-3]} {v}" for k, v in r.items() if k.endswith("_us") and k != "best_us")
            print(f"| small | n={r['n']}: {paths} (us) | {r['B']} | {r['auto_us'] / 1e3:.4f} | "
                  f"{round(r['B'] / (r['auto_us'] * 1e-6), 1)} | - | {r['auto_frac_8TBs']} |", file=sys.stderr)
            continue
        elif r["sweep"] == "shapes":
            print(f"| shapes | {r['workload']} quantize | {r['B']} | {r['quantize_ms']} | - | {r['quantize_GBs']} | "
                  f"{r['quantize_frac_8TBs']} |", file=sys.stderr)
            print(f"| shapes | {r['workload']} decode | {r['B']} | {r['decode_ms']} | {r['decode_seq_steps_per_s']} | "
                  f"{r['decode_GBs']} | {r['decode_frac_8TBs']} |", file=sys.stderr)
            continue
        else:
            pt, ms = f"{r['budget_GiB']} GiB, n={r['n']}, {r['cache']}", r["step_ms"]
        print(f"| {r['sweep']} | {pt} | {r['B']} | {ms} | {r['seq_steps_per_s']} | {r['GBs']} | {r['frac_8TBs']} |",
              file=sys.stderr)


# ---------------------------------------------------------------------------
# rocprofv3 summaries -> profiles/
# ---------------------------------------------------------------------------

def _rows(pattern):
    rows = []
    for f in glob.glob(pattern, recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize(dirs, workload, command_note, profile_name=None):
    """Write profiles/<kernel>_<workload>.md from kernel-trace stats and
    counter CSVs, and profiles/traffic_<workload>.json with HBM bytes per launch
    scaled by the copy-kernel reference."""
    os.makedirs(PROFILES, exist_ok=True)
    stats = []
    for d in dirs:
        stats += _rows(os.path.join(d, "**", "*kernel_stats.csv"))
    counters = []
    for d in dirs:
        counters += _rows(os.path.join(d, "**", "*counter_collection.csv"))
    lines = [f"# rocprofv3 summary — {workload}", "", "Commands:", "", "```", command_note.strip(), "```", ""]
    if stats:
        lines += ["## Kernel stats (--kernel-trace --stats)", "",
                  "| kernel | calls | avg (us) | total (ms) | % |", "|---|---|---|---|---|"]
        for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0))):
            lines.append(f"| {r['Name'][:90]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r.get('Percentage', 0)):.1f} |")
        lines.append("")
    traffic = {}
    if counters:
        per = {}
        for r in counters:
            name = r.get("Kernel_Name", r.get("Kernel-Name", ""))
            cname = r.get("Counter_Name", r.get("Counter-Name", ""))
            val = float(r.get("Counter_Value", r.get("Counter-Value", 0)))
            per.setdefault((name, cname), []).append(val)
        lines += ["## Counters (--pmc, per dispatch, averaged; FETCH_SIZE / WRITE_SIZE in KiB)", "",
                  "| kernel | counter | dispatches | avg |", "|---|---|---|---|"]
        for (name, cname), vals in sorted(per.items()):
            lines.append(f"| {name[:80]} | {cname} | {len(vals)} | {sum(vals) / len(vals):.1f} |")
        lines.append("")
        copy_read = [v for (n_, c), vs in per.items() if "neg" in n_.lower() and c == "FETCH_SIZE" for v in vs]
        copy_write = [v for (n_, c), vs in per.items() if "neg" in n_.lower() and c == "WRITE_SIZE" for v in vs]
        ref_bytes = (1 << 29) * 2
        f_read = (sum(copy_read) / len(copy_read) * 1024 / ref_bytes) if copy_read else None
        f_write = (sum(copy_write) / len(copy_write) * 1024 / ref_bytes) if copy_write else None
        if f_read or f_write:
            lines += [f"Copy-kernel reference (1 GiB read + 1 GiB written): FETCH_SIZE factor "
                      f"{f_read}, WRITE_SIZE factor {f_write} (counter KiB x 1024 / true bytes).", ""]

        def op_bytes(kernels):
            # one call launches each kernel in `kernels` once: sum their per-dispatch averages
            tot = 0.0
            for cname, fac in (("FETCH_SIZE", f_read), ("WRITE_SIZE", f_write)):
                for kern in kernels:
                    vals = [v for (n_, c), vs in per.items() if c == cname and kern in n_ for v in vs]
                    if not vals or not fac:
                        return None
                    tot += sum(vals) / len(vals) * 1024 / fac
            return tot
        for op, kernels in (("quantize", ("qf_init", "qf_b1")), ("decode", ("df_b1",))):
            b = op_bytes(kernels)
            if b is not None:
                traffic[op] = {"bytes_per_launch": round(b), "kernels": list(kernels),
                               "source_digest": source_digest(*KERNEL_SOURCES[op])}
    name = profile_name or ("summary" if not stats else "kernels")
    with open(os.path.join(PROFILES, f"{name}_{workload}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    if traffic:
        with open(os.path.join(PROFILES, f"traffic_{workload}.json"), "w") as fh:
            json.dump(traffic, fh, indent=1)
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_n8192")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["step", "decode", "copy"], default=None)
    ap.add_argument("--path", default="auto", choices=["auto", "fast", "fast_one", "fast_lds", "fast_pipe", "fast_split",
                                                       "fast_wide", "generic"],
                    help="decode schedule for --only decode")
    ap.add_argument("--summarize", nargs="+", default=None, metavar="DIR")
    ap.add_argument("--sweeps", nargs="*", choices=["bits", "budget", "graph", "stream", "tail", "shapes", "small"],
                    default=None)
    ap.add_argument("--command-note", default="")
    ap.add_argument("--profile-name", default=None, help="profiles/<name>_<workload>.md for --summarize")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload, args.command_note, args.profile_name)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path shards by batch or kv head with no "
              "communication, and no multi-GPU figure is produced. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweeps is not None:
        sweeps(args)
        return
    run(args)


if __name__ == "__main__":
    main()
