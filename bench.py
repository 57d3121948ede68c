#!/usr/bin/env python3
"""Throughput of QuaRot's 4-bit linear-layer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input,
launched in order on one HIP stream:
  qr_rotate_quant  x [M, K] fp16 -> int4 codes + per-token (or group) scales
  qr_int4_gemm     codes x pre-rotated int4 weights -> y [M, N] fp16
  qr_kv_quant      the new K and V rows (c2: the K and V heads of the fused
                   QKV output; c5: the decode step's K and V rows)
Workloads (--config; the layer shapes of the QuaRot summary's LLaMA-2 7B/70B
blocks at batch 64 x sequence 2048, "Key points"):
  c3 (default)  LLaMA-2-7B down_proj: x 131072 x 11008 -> 4096, rotation
                (H_64/8) kron O_172, per-token / per-channel int4
  c2            LLaMA-2-7B fused QKV prefill: x 2048 x 4096 -> 12288,
                D.H_4096, per-token / per-channel, plus KV quant of K and V
  c4            LLaMA-2-70B MLP up/gate: x 16384 x 8192 -> 28672, D.H_8192,
                group 128 on both sides
  c5            decode step at batch 64: x 64 x 4096 -> 4096 (memory-bound
                GEMM) plus KV quant of 64 tokens x 32 heads of K and V
Inputs are synthetic and seeded (package ``workloads``) and resident in HBM
before timing; weights are prepared on the GPU before timing (rotate +
quantize the rows of W^T with the same library call).  Steps cycle over enough
distinct buffer sets (>= 1 GiB, at least two) that nothing is served from the
256 MB Infinity Cache between uses, and consecutive steps alternate over
HIP streams of default priority (--streams; a buffer set is reused only after
the step that last used it has finished: an event dependency).

Prints one JSON line.  `value` is whole-step throughput in TOPS (2 M N K per
step).  Per-kernel times are medians of >= 20 HIP event pairs recorded
around single launches on the launch stream.  `roofline` is for the
dominant kernel of the step; `cpu_baseline` is the CPU oracle timed on a
bounded row sample of the same workload and extrapolated to the whole step;
`peaks_measured` holds what this GPU attains for a streaming copy and for
back-to-back int8 / fp16 MFMAs (include/qr_peaks.h), the second denominators.

  python bench.py [--config c3] [--steps K] [--warmup W] [--streams N] [--graph 0|1] [--no-cpu]
  python bench.py --suite [--only case,...]      # every kernel at every shape
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published (5.0 POP/s)
FP16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16 MFMA, published (2.5 PFLOP/s)
CACHE_BYTES = 1 << 30        # cycle buffers over >= 1 GiB (MALL is 256 MB)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
STEP_CONFIGS = ("c3", "c2", "c4", "c5")
# Steps alternate over this many HIP streams unless --streams says otherwise:
# overlapping consecutive steps helps c2's short launches (104 vs 108-109 us
# per step), costs ~2% at c3 (5.64 vs 5.75-5.78 ms), where each kernel fills
# the GPU by itself, and costs c5 15-20% (21.3 vs 25.2-26.6 us): the decode
# step is bound by the host's ~7 us per launch call, and the second stream
# adds event bookkeeping on the host every step.
DEFAULT_STREAMS = {"c3": 1, "c4": 1, "c2": 2, "c5": 1}
# Timed and warm-up steps by default: the short steps of c2 (~0.1 ms) and c5
# (~20 us) need many more of them than c3 and c4 (~5 ms) for a timed region
# that a pair of events measures well (20 decode steps gave 35.8 us per step
# where 200 gave 21.3).
DEFAULT_STEPS = {"c3": (20, 5), "c4": (20, 5), "c2": (200, 20), "c5": (500, 50)}
# --graph 1 replays each step from a HIP graph captured per buffer set.  It
# is off by default: the decode step took 55-57 us per step from graphs
# against 35-38 us launched kernel by kernel (c2: no difference).
DEFAULT_GRAPH = {"c3": 0, "c4": 0, "c2": 0, "c5": 0}
# token rows of the CPU oracle sample per config (one pass takes ~0.05-7 s on
# 16 cores); passes repeat until CPU_MIN_SECONDS of oracle work are timed
CPU_ROWS = {"c2": 2048, "c3": 2048, "c4": 512, "c5": 64}
CPU_MIN_SECONDS = 10.0
METRIC = "rotate+quant+int4 GEMM TOPS and GB/s at 7B/70B layer shapes; % of roofline"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (0: the config's default)")
    ap.add_argument("--warmup", type=int, default=-1, help="untimed steps first (-1: the config's default)")
    ap.add_argument("--config", default="c3", choices=STEP_CONFIGS)
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--graph", type=int, default=-1, choices=(-1, 0, 1),
                    help="1: replay each step from a HIP graph captured per buffer set; 0: launch its kernels "
                         "one by one; -1: the config's default")
    ap.add_argument("--cpu-rows", type=int, default=0, help="token rows in the CPU oracle sample (0 = default)")
    ap.add_argument("--streams", type=int, default=0,
                    help="HIP streams the steps alternate over (1: strictly one step after another; 0: the "
                         "workload's default, 2 for the short c2 step whose launches gain from overlapping, "
                         "1 for c3 and c4 whose kernels each fill the GPU and for c5 whose step is bound "
                         "by the host's launch calls)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="also run one probe copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to cycle (0 = enough for 1 GiB, >= 2)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the step, time each kernel at every config's shape (one JSON line each)")
    ap.add_argument("--only", default="", help="with --suite: comma-separated case names to run")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read rocprofv3 FETCH_SIZE / WRITE_SIZE runs of `bench.py --config C --copy-calib MIB` "
                         "and add the dominant kernel's HBM bytes per launch to profiles/traffic.json")
    ap.add_argument("--calib-mib", type=int, default=1024, help="size of the copy used with --ingest-pmc")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="digest a rocprofv3 kernel trace of this script (per kernel, all dispatches and the "
                         "last --trace-last ones) and exit")
    ap.add_argument("--trace-last", type=int, default=20, help="dispatches of the per-launch timing phase")
    ap.add_argument("--codes-sweep", action="store_true",
                    help="the config's int4 GEMM looped ~2 s each on constant, workload and uniformly random "
                         "codes, then its rotate-quant on a constant and on the workload input, with the shader "
                         "clock sampled by rocm-smi meanwhile (one JSON line per case)")
    return ap.parse_args()


# ---------------------------------------------------------------- helpers

def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


CSRC = "rotation_bit_quantized_amd/csrc/"
KERNEL_SOURCES = {
    "gemm_prefill_kernel": [CSRC + "gemm_prefill.hip", CSRC + "qr_common.h"],
    "gemm_decode_lds_kernel": [CSRC + "gemm_decode.hip", CSRC + "qr_common.h"],
    "rq_kron_kernel": [CSRC + "rq_kron.hip", CSRC + "qr_common.h"],
    "rq_pow2_kernel": [CSRC + "rq_pow2.hip", CSRC + "qr_common.h"],
    "kv_quant_kernel": [CSRC + "kv_quant.hip", CSRC + "qr_common.h"],
}


def load_traffic(key, kernel, algorithmic_bytes):
    """HBM bytes of one launch from committed rocprofv3 counter runs, or None
    when they are missing or the kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
            "total_bytes": rec["fetch_bytes"] + rec["write_bytes"], "algorithmic_bytes": algorithmic_bytes,
            "calibration": rec.get("calibration")}


def time_each(fn, n, stream, warm=3):
    """Median and mean duration (ms) of one launch of fn(i): a HIP event pair
    on the launch stream around each of n launches (the per-dispatch span,
    as a kernel trace reports it)."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    return statistics.median(t), sum(t) / len(t)


def measure_peaks(dev):
    """Attainable rates on this GPU: a 2 x 1 GiB streaming copy, and back-to-
    back int8 and fp16 MFMAs (medians of 5 launches each)."""
    import torch
    import rotation_bit_quantized_amd as qr
    st = torch.cuda.current_stream()
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    src.fill_(1)
    copy_ms, _ = time_each(lambda i: qr.peak_copy(src, dst), 5, st, warm=1)
    del src, dst
    out = {"hbm_copy_GBs": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1)}
    for kind, key in ((0, "mfma_int8_TOPS"), (3, "mfma_int8_16x16_TOPS"), (1, "mfma_fp16_16x16_TFLOPS"),
                      (2, "mfma_fp16_32x32_TFLOPS")):
        buf, ops = qr.peak_mfma(kind, 20000)
        ms, _ = time_each(lambda i: qr.peak_mfma(kind, 20000, buf), 5, st, warm=1)
        out[key] = round(ops / (ms * 1e-3) / 1e12, 1)
    out["how"] = ("qr_peak_copy of 1 GiB (2 GiB moved); qr_peak_mfma: 8 waves per CU, four independent "
                  "v_mfma_i32_32x32x32_i8 / v_mfma_i32_16x16x64_i8 / v_mfma_f32_16x16x32_f16 / v_mfma_f32_32x32x16_f16 "
                  "chains, "
                  "20000 rounds; medians of 5")
    return out


def measure_codes_peak(a_codes, w_codes, stream, seconds=0.5):
    """The int8 MFMA loop of qr_peak_mfma_codes on the step's own activation
    and weight codes, run for about `seconds` so that the clock has settled
    to what this operand data draws (it drops within ~0.1-0.4 s of dense
    MFMA work); median of the second half of the calls."""
    import rotation_bit_quantized_amd as qr
    a = a_codes.reshape(-1)
    w = w_codes.reshape(-1)
    a = a[: a.numel() // 16 * 16]
    w = w[: w.numel() // 16 * 16]
    iters = 20000                                   # ~20 ms per call
    buf, ops = qr.peak_mfma_codes(a, w, iters)
    times, t0 = [], time.perf_counter()
    while time.perf_counter() - t0 < seconds or len(times) < 10:
        ms, _ = time_each(lambda i: qr.peak_mfma_codes(a, w, iters, buf), 1, stream, warm=0)
        times.append(ms)
    return round(ops / (statistics.median(times[len(times) // 2:]) * 1e-3) / 1e12, 1)


# ---------------------------------------------------------------- the oracle on a row sample

def oracle_rows_rotated(x, cfg, signs, dense):
    """y = x R with the oracle's pinned routines (fwht for D.H_n, rotate_kron for
    the Kronecker rotation)."""
    import oracle as O
    if cfg.dense_m > 1:
        return O.rotate_kron(x, cfg.had_n, dense.astype(np.float64), signs)
    d = np.ones(cfg.K) if signs is None else np.asarray(signs, np.float64)
    return O.fwht(np.asarray(x, np.float64) * d) / np.sqrt(cfg.K)


def cpu_baseline(cfg, rows, kv_rows):
    """The oracle on a bounded sample: `rows` token rows through rotate,
    quantize, int64 GEMM against all N output channels and fp64 dequantize,
    plus the KV quantizer on those rows' K and V (c2, c5).  The pass is
    repeated, each time from the input, until at least CPU_MIN_SECONDS of
    work have been timed.  Weight preparation (offline in the method) is not
    timed.  Throughput is extrapolated linearly to the whole step (every
    stage is per token)."""
    import oracle as O
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    x = W.make_x(cfg, rows=np.arange(rows))
    w = W.make_w(cfg)
    signs, dense = W.make_signs(cfg), W.make_dense(cfg)
    wr = oracle_rows_rotated(np.ascontiguousarray(w.T), cfg, signs, dense).T      # R^T W
    qw, sw = O.quantize_weights(wr, cfg.group)
    blocks = np.array_split(np.arange(cfg.N), threads)
    passes = 0
    t0 = time.perf_counter()
    while True:
        y = oracle_rows_rotated(x, cfg, signs, dense)
        qx, sx, _ = O.quantize_symmetric(y, cfg.group)
        with cf.ThreadPoolExecutor(threads) as ex:
            parts = list(ex.map(lambda b: O.int_gemm(qx, qw[b], cfg.group), blocks))
        acc = np.concatenate(parts, axis=-1)
        out = O.dequantize_output(acc, sx, sw, cfg.group)
        if kv_rows is not None:
            for t in kv_rows(out):
                O.kv_quantize(t)
        passes += 1
        if time.perf_counter() - t0 >= CPU_MIN_SECONDS:
            break
    dt = time.perf_counter() - t0
    ops = 2.0 * rows * cfg.N * cfg.K * passes
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "passes": passes,
            "sample": f"{rows} of {cfg.M} token rows, {passes} timed passes (rate extrapolated linearly to the whole step): fp64 "
                      f"rotation ({'rotate_kron' if cfg.dense_m > 1 else 'fwht'}), RTN, int64 GEMM against all "
                      f"{cfg.N} channels (column blocks over {threads} threads), fp64 dequant"
                      + (", KV quant of the sampled rows' K and V" if kv_rows is not None else "")
                      + "; weight prep untimed"}


# ---------------------------------------------------------------- counters

def ingest_pmc(cfg_name, fetch_dir, write_dir, calib_mib):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the step's GEMM, of its
    rotate-quant kernel and (c2, c5) of its KV quantizer, and of the
    calibration copy; scale each kernel's by
    known/measured of the copy (a copy of B bytes reads B and writes B).  The
    median over a kernel's dispatches is taken, so the one weight-preparation
    launch of the rotate-quant kernel (another row count) does not count."""
    import csv
    import glob
    import re
    gemm = "gemm_decode_lds_kernel" if cfg_name == "c5" else "gemm_prefill_kernel"
    cfg = None
    try:
        import workloads as W
        cfg = W.CONFIGS[cfg_name]
    except Exception:
        pass
    rq = "rq_kron_kernel" if cfg is not None and cfg.dense_m > 1 else "rq_pow2_kernel"

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] == counter:
                    key = (row["Dispatch_Id"], row["Kernel_Name"])
                    vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        return vals

    def kernel_median(vals, kernel):
        v = [x for (d, k), x in vals.items() if kernel in k]
        if not v:
            raise SystemExit(f"no {kernel} dispatches in the counter data")
        return statistics.median(v), len(v), [k for (d, k) in vals if kernel in k][0]

    def copy_max(vals):
        v = [x for (d, k), x in vals.items() if "peak_copy" in k]
        if not v:
            raise SystemExit("no probe copy dispatch in the counter data")
        return max(v)

    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    known_kib = calib_mib * 1024.0
    f_scale = known_kib / copy_max(fetch)
    w_scale = known_kib / copy_max(write)
    try:
        recs = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        recs = {}
    kinds = [(f"int4_gemm_{cfg_name}", gemm), (f"rotate_quant_{cfg_name}", rq)]
    if any("kv_quant_kernel" in k for (d, k) in fetch):
        kinds.append((f"kv_quant_{cfg_name}", "kv_quant_kernel"))
    for key, kernel in kinds:
        k_fetch, n, kname = kernel_median(fetch, kernel)
        k_write, _, _ = kernel_median(write, kernel)
        m = re.search(kernel + r"<[^>]*>", kname)
        recs[key] = {
            "kernel": m.group(0) if m else kernel, "source_hash": source_hash(KERNEL_SOURCES[kernel]),
            "fetch_bytes": round(k_fetch * 1024 * f_scale), "write_bytes": round(k_write * 1024 * w_scale),
            "dispatches": n,
            "calibration": {"copy": f"qr_peak_copy of {calib_mib} MiB (largest copy dispatch)",
                            "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                            "raw_fetch_kib": round(k_fetch, 1), "raw_write_kib": round(k_write, 1)},
            "command": f"rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py "
                       f"--config {cfg_name} --steps 3 --warmup 1 --no-cpu --no-peaks --copy-calib {calib_mib}"}
        print(json.dumps({key: recs[key]}))
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(recs, open(TRAFFIC_FILE, "w"), indent=1)


def trace_summary(path, last):
    """Digest of a rocprofv3 kernel trace (``*_kernel_trace.csv``): per kernel,
    the calls, mean / min / max duration over all dispatches, and mean and
    median over its last `last` dispatches (the per-launch timing phase that
    follows the timed steps)."""
    import csv
    import re
    per = {}
    for row in csv.DictReader(open(path)):
        name = row["Kernel_Name"]
        name = re.sub(r"^void ", "", name)
        name = re.sub(r"\(anonymous namespace\)::", "", name)
        name = re.sub(r"\((?!anonymous).*$", "", name)
        per.setdefault(name, []).append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))
    lines = [f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'lastN':>6} {'lastN_avg':>10} "
             f"{'lastN_med':>10}  kernel"]
    order = sorted(per.items(), key=lambda kv: -sum(e - s for s, e in kv[1]))
    for name, spans in order:
        spans.sort()
        d = [(e - s) / 1e3 for s, e in spans]
        tail = d[-last:] if len(d) >= last else []
        lines.append(f"{len(d):>6} {sum(d) / len(d):>10.1f} {min(d):>10.1f} {max(d):>10.1f} "
                     f"{len(tail) or '-':>6} "
                     + (f"{sum(tail) / len(tail):>10.1f} {statistics.median(tail):>10.1f}" if tail
                        else f"{'-':>10} {'-':>10}") + f"  {name[:100]}")
    print("\n".join(lines))


# ---------------------------------------------------------------- the step

def run_step(args):
    import torch
    import workloads as W
    import rotation_bit_quantized_amd as qr

    qr.library()                     # no fallback: fail loudly without the HIP library
    cfg = W.CONFIGS[args.config]
    M, N, K, group = cfg.M, cfg.N, cfg.K, cfg.group
    G = 1 if group == 0 else K // group
    if args.steps <= 0:
        args.steps = DEFAULT_STEPS[cfg.name][0]
    if args.warmup < 0:
        args.warmup = DEFAULT_STEPS[cfg.name][1]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    peaks = None if args.no_peaks else measure_peaks(dev)

    # ------------------------------------------------------ resident inputs (untimed)
    signs, dense = W.make_signs(cfg), W.make_dense(cfg)
    rot = (qr.Rotation.kronecker(cfg.had_n, dense, signs) if cfg.dense_m > 1
           else qr.Rotation.hadamard(K, signs))
    wt = torch.from_numpy(np.ascontiguousarray(W.make_w(cfg).T)).to(dev)
    wc0, ws0 = qr.rotate_quant(wt, rot, group)          # offline weight prep, on the GPU
    del wt
    x0 = torch.from_numpy(W.make_x(cfg)).to(dev)
    # KV rows of the step: c2 quantizes the K and V heads of its own fused QKV
    # output in place; c5 quantizes the decode step's new K and V rows
    if args.config == "c2":
        H = K // 128
        kv_T, kv_H = M, 2 * H
    elif args.config == "c5":
        k_host, v_host = W.make_kv(cfg)
        kv_T, kv_H = k_host.shape[0], 2 * k_host.shape[1]
        kv0 = torch.from_numpy(np.ascontiguousarray(np.concatenate([k_host, v_host], axis=1))).to(dev)
    else:
        kv_T = kv_H = 0
    has_kv = kv_T > 0
    set_bytes = (x0.numel() * 2 + M * K // 2 + M * G * 4 + wc0.numel() + ws0.numel() * 4 + M * N * 2
                 + kv_T * kv_H * (64 + 5) + (kv_T * kv_H * 256 if args.config == "c5" else 0))
    nsets = args.sets or max(2, -(-CACHE_BYTES // set_bytes))
    sets = []
    for i in range(nsets):
        s = dict(x=x0 if i == 0 else x0.clone(), wc=wc0 if i == 0 else wc0.clone(),
                 ws=ws0 if i == 0 else ws0.clone(),
                 xc=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                 xs=torch.empty((M,) if group == 0 else (M, G), dtype=torch.float32, device=dev),
                 y=torch.empty((M, N), dtype=torch.float16, device=dev))
        if has_kv:
            s["kvc"] = torch.empty((kv_T, kv_H, 64), dtype=torch.uint8, device=dev)
            s["kvs"] = torch.empty((kv_T, kv_H), dtype=torch.float32, device=dev)
            s["kvz"] = torch.empty((kv_T, kv_H), dtype=torch.uint8, device=dev)
            if args.config == "c5":
                s["kv"] = kv0 if i == 0 else kv0.clone()
        sets.append(s)
    del x0, wc0, ws0
    nstreams = args.streams if args.streams > 0 else DEFAULT_STREAMS[cfg.name]
    streams = [stream] + [torch.cuda.Stream(device=dev) for _ in range(max(1, nstreams) - 1)]

    def rq(s, st=stream):
        qr.rotate_quant(s["x"], rot, group, codes=s["xc"], scales=s["xs"], stream=st)

    def gemm(s, st=stream):
        qr.int4_gemm(s["xc"], s["xs"], s["wc"], s["ws"], group, y=s["y"], stream=st)

    def kv(s, st=stream):
        # one launch over every K and V head vector of the step's tokens
        src = s["y"][:, K:3 * K] if args.config == "c2" else s["kv"]
        qr.kv_quant(src, codes=s["kvc"], scales=s["kvs"], zeros=s["kvz"], stream=st)

    use_graph = (args.graph if args.graph >= 0 else DEFAULT_GRAPH[cfg.name]) == 1
    if use_graph:
        # one graph per buffer set, captured after one eager pass (which sets
        # up the library's per-process state); the step's kernels write only
        # their outputs, so a replay recomputes the whole step
        for s in sets:
            rq(s)
            gemm(s)
            if has_kv:
                kv(s)
        torch.cuda.synchronize()
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream()
                rq(s, cs)
                gemm(s, cs)
                if has_kv:
                    kv(s, cs)
            s["graph"] = g
        torch.cuda.synchronize()

    def step(i):
        s = sets[i % nsets]
        st = streams[i % len(streams)]
        if "done" in s and s["done_on"] is not st:
            st.wait_event(s["done"])   # the set's previous step, on another stream, has finished
        if use_graph:
            with torch.cuda.stream(st):
                s["graph"].replay()
        else:
            rq(s, st)
            gemm(s, st)
            if has_kv:
                kv(s, st)
        if len(streams) > 1:
            s["done"] = torch.cuda.Event()
            s["done"].record(st)
            s["done_on"] = st

    def fork():
        ev = torch.cuda.Event()
        ev.record(stream)
        for st in streams[1:]:
            st.wait_event(ev)

    def join():
        for st in streams[1:]:
            ev = torch.cuda.Event()
            ev.record(st)
            stream.wait_event(ev)

    if args.copy_calib:   # a copy of known size for the HBM counter calibration
        nb = args.copy_calib << 20
        a = torch.ones(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        qr.peak_copy(a, b)
        torch.cuda.synchronize()
        del a, b

    fork()
    for i in range(args.warmup):
        step(i)
    join()
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps, nothing else on the streams
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    fork()
    for i in range(args.steps):
        step(i)
    join()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps

    # per-kernel durations (after the timed region, same stream, rotating
    # buffer sets): medians of HIP event pairs around single launches
    nrep = max(20, args.steps)
    rq_ms, rq_mean = time_each(lambda i: rq(sets[i % nsets]), nrep, stream)
    gemm_ms, gemm_mean = time_each(lambda i: gemm(sets[i % nsets]), nrep, stream)
    kv_ms = time_each(lambda i: kv(sets[i % nsets]), nrep, stream) if has_kv else None

    # the int8 MFMA rate attainable on this step's own codes (prefill)
    if peaks and M > 64:
        peaks["mfma_int8_codes_TOPS"] = measure_codes_peak(sets[0]["xc"], sets[0]["wc"], stream)
        peaks["how_codes"] = ("qr_peak_mfma_codes: the kind-0 loop on operands widened from the step's activation "
                              "codes (A) and weight codes (W), run ~0.5 s so that the clock settles; median of "
                              "the second half of ~20 ms calls")

    ops = 2.0 * M * N * K
    value = ops / (ms_per_step * 1e-3) / 1e12
    rq_bytes = M * K * 2 + M * K // 2 + M * G * 4
    gemm_bytes = M * K // 2 + N * K // 2 + M * N * 2 + 4 * G * (M + N)
    kv_bytes = kv_T * kv_H * (256 + 64 + 5)
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    gemm_gbs = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    rq_gbs = rq_bytes / (rq_ms * 1e-3) / 1e9

    def frac(v, peak, key):
        d = {"frac_peak": round(v / peak, 4)}
        if peaks:
            d["frac_measured_peak"] = round(v / peaks[key], 4)
        return d

    kernels = {
        "rotate_quant": {"kernel": "rq_kron_kernel" if cfg.dense_m > 1 else "rq_pow2_kernel",
                         "us_median": round(rq_ms * 1e3, 3), "us_mean": round(rq_mean * 1e3, 3),
                         "GB/s": round(rq_gbs, 1), **frac(rq_gbs, HBM_PEAK_GBS, "hbm_copy_GBs"),
                         "bytes": rq_bytes},
        "int4_gemm": {"kernel": "gemm_decode_lds_kernel" if M <= 64 else "gemm_prefill_kernel",
                      "us_median": round(gemm_ms * 1e3, 3), "us_mean": round(gemm_mean * 1e3, 3),
                      "TOPS": round(gemm_tops, 2), **frac(gemm_tops, INT8_PEAK_TOPS, "mfma_int8_TOPS"),
                      **({"frac_measured_codes_peak": round(gemm_tops / peaks["mfma_int8_codes_TOPS"], 4)}
                         if peaks and "mfma_int8_codes_TOPS" in peaks else {}),
                      "GB/s": round(gemm_gbs, 1), "frac_hbm": round(gemm_gbs / HBM_PEAK_GBS, 4),
                      "bytes": gemm_bytes},
    }
    if cfg.dense_m > 1:
        # the dense factor is a second, MFMA-side ceiling of the Kronecker rotation
        dflops = 2.0 * M * K * cfg.dense_m
        kernels["rotate_quant"]["dense_TFLOPS"] = round(dflops / (rq_ms * 1e-3) / 1e12, 1)
    if has_kv:
        kv_gbs = kv_bytes / (kv_ms[0] * 1e-3) / 1e9
        kernels["kv_quant"] = {"kernel": "kv_quant_kernel", "vectors": [kv_T, kv_H],
                               "us_median": round(kv_ms[0] * 1e3, 3), "us_mean": round(kv_ms[1] * 1e3, 3),
                               "GB/s": round(kv_gbs, 1), **frac(kv_gbs, HBM_PEAK_GBS, "hbm_copy_GBs"),
                               "bytes": kv_bytes}

    # the dominant kernel of the step and its roofline
    if M <= 64:   # decode: the GEMM streams the weights, HBM-bound
        traffic = load_traffic(f"int4_gemm_{cfg.name}", "gemm_decode_lds_kernel", gemm_bytes)
        roofline = {"bound": "hbm", "kernel": "int4_gemm (gemm_decode_lds_kernel)", "achieved": round(gemm_gbs, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gemm_gbs / HBM_PEAK_GBS, 4)}
    else:
        traffic = load_traffic(f"int4_gemm_{cfg.name}", "gemm_prefill_kernel", gemm_bytes)
        roofline = {"bound": "mfma", "kernel": "int4_gemm (gemm_prefill_kernel)", "achieved": round(gemm_tops, 2),
                    "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4)}
        if peaks and "mfma_int8_codes_TOPS" in peaks:
            # what the int8 MFMAs attain on this step's own codes (the clock under dense MFMA work falls as
            # more operand bits toggle): the data-matched ceiling beside the datasheet one
            roofline["peak_measured_on_codes"] = peaks["mfma_int8_codes_TOPS"]
            roofline["frac_of_measured_on_codes"] = round(gemm_tops / peaks["mfma_int8_codes_TOPS"], 4)
    roofline["traffic"] = None if traffic is None else traffic["total_bytes"]
    roofline["traffic_detail"] = traffic
    roofline["achieved_from"] = "median of per-launch HIP event pairs on the launch stream"

    rot_desc = (f"(H_{cfg.had_n}/{int(np.sqrt(cfg.had_n))}) kron O_{cfg.dense_m}" if cfg.dense_m > 1
                else f"D.H_{K}/{np.sqrt(K):g}")
    quant_desc = "per-token / per-channel int4" if group == 0 else f"int4 with group {group} on both sides"
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.desc}; rotate {rot_desc} + {quant_desc} RTN, int4 GEMM (int8 MFMA, "
                        f"fp16 out)" + (f", 4-bit KV quant of {kv_T} tokens x {kv_H} K/V heads" if has_kv else ""),
            "M": M, "N": N, "K": K, "group": group, "codes": "int4", "mfma": "int8 -> int32",
            "rotation": rot_desc, "buffer_sets": nsets, "streams": len(streams), "graph": use_graph,
        },
        "kernels": kernels,
        "roofline": roofline,
        "wall_s": round(wall, 4),
    }
    if peaks:
        out["peaks_measured"] = peaks
    if not args.no_cpu:
        rows = min(args.cpu_rows or CPU_ROWS[cfg.name], M)
        kv_rows = None
        if args.config == "c2":
            kv_rows = lambda y: [y[:, K:2 * K].astype(np.float16).reshape(-1, K // 128, 128),
                                 y[:, 2 * K:3 * K].astype(np.float16).reshape(-1, K // 128, 128)]
        elif args.config == "c5":
            kv_rows = lambda y: [k_host[:rows], v_host[:rows]]
        out["cpu_baseline"] = cpu_baseline(cfg, rows, kv_rows)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- clock vs operand data

def sclk_mhz():
    """Current shader clock from rocm-smi (None if it cannot be read)."""
    import re
    import subprocess
    try:
        txt = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    m = re.search(r"sclk clock level:[^(]*\((\d+)Mhz\)", txt)
    return int(m.group(1)) if m else None


def codes_sweep(args):
    """The same GEMM launch on three kinds of operand data, then the same
    rotate-quant launch on two inputs.  The instruction stream is identical;
    only the bits the MFMAs toggle differ, and with them the clock this part
    sustains under the kernel."""
    import threading
    import torch
    import workloads as W
    import rotation_bit_quantized_amd as qr
    qr.library()
    cfg = W.CONFIGS[args.config]
    M, N, K, group = cfg.M, cfg.N, cfg.K, cfg.group
    if M <= 64:
        raise SystemExit("--codes-sweep is for the prefill configs")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    signs, dense = W.make_signs(cfg), W.make_dense(cfg)
    rot = (qr.Rotation.kronecker(cfg.had_n, dense, signs) if cfg.dense_m > 1 else qr.Rotation.hadamard(K, signs))
    wt = torch.from_numpy(np.ascontiguousarray(W.make_w(cfg).T)).to(dev)
    wc, ws = qr.rotate_quant(wt, rot, group)
    del wt
    x = torch.from_numpy(W.make_x(cfg)).to(dev)
    xc, xs = qr.rotate_quant(x, rot, group)
    del x
    y = torch.empty((M, N), dtype=torch.float16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    kinds = [("constant", torch.full_like(xc, 0x35), torch.full_like(wc, 0x17)),
             ("workload", xc, wc),
             ("uniform", torch.randint(0, 256, xc.shape, dtype=torch.uint8, device=dev, generator=g),
              torch.randint(0, 256, wc.shape, dtype=torch.uint8, device=dev, generator=g))]

    def looped(name, fn, ops, what):
        fn()
        torch.cuda.synchronize()
        clocks, stop = [], threading.Event()

        def sample():
            while not stop.wait(0.25):
                c = sclk_mhz()
                if c is not None:
                    clocks.append(c)
        th = threading.Thread(target=sample)
        th.start()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0, n = time.perf_counter(), 0
        e0.record()
        while time.perf_counter() - t0 < 2.0:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            n += 10
        e1.record()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        us = e0.elapsed_time(e1) * 1e3 / n
        late = clocks[len(clocks) // 3:]
        print(json.dumps({"kernel": what, "data": name, "config": cfg.name, "launches": n,
                          "us_per_launch": round(us, 1), **ops(us),
                          "sclk_MHz_median": statistics.median(late) if late else None,
                          "sclk_samples": len(clocks)}), flush=True)
        time.sleep(1.0)

    for name, a, w in kinds:
        looped(name, lambda: qr.int4_gemm(a, xs, w, ws, group, y=y),
               lambda us: {"TOPS": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 1)}, "int4_gemm")
    # the rotate-quant kernel on the step's input and on a constant input
    x = torch.from_numpy(W.make_x(cfg)).to(dev)
    rq_bytes = M * K * 2 + M * K // 2 + M * (1 if group == 0 else K // group) * 4
    for name, xx in (("constant", torch.full_like(x, 0.25)), ("workload", x)):
        looped(name, lambda: qr.rotate_quant(xx, rot, group, xc, xs),
               lambda us: {"GBs": round(rq_bytes / (us * 1e-6) / 1e9, 1)}, "rotate_quant")


# ---------------------------------------------------------------- per-kernel suite

def suite(args):
    """Kernel-level throughput at each config's shape: medians of >= 20 HIP
    event pairs around single launches.  Inputs cycle over >= 1 GiB of
    distinct buffers (weights included), so what a launch touches comes from
    HBM, not the 256 MB Infinity Cache, unless the case is a single-shot
    latency case (then said so in its line)."""
    import torch
    import workloads as W
    import rotation_bit_quantized_amd as qr
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream()
    only = set(filter(None, args.only.split(",")))
    g = torch.Generator(device=dev)
    g.manual_seed(1234)

    def codes(rows, k):
        return torch.randint(0, 256, (rows, k // 2), dtype=torch.uint8, device=dev, generator=g)

    def emit(case, **kw):
        print(json.dumps({"case": case, **kw}), flush=True)

    def copies(make, per_bytes):
        n = max(2, -(-CACHE_BYTES // max(1, per_bytes)))
        return [make() for _ in range(n)]

    def med(fn, reps):
        return time_each(fn, max(20, reps), st)[0]

    def rq_case(name, cfg, rows, group, reps=20):
        if only and name not in only:
            return
        c = W.CONFIGS[cfg]
        x = torch.from_numpy(W.make_x(c, rows=np.arange(rows))).to(dev)
        if c.dense_m > 1:
            rot = qr.Rotation.kronecker(c.had_n, W.make_dense(c), W.make_signs(c))
        else:
            rot = qr.Rotation.hadamard(c.K, W.make_signs(c))
        nbytes = rows * c.K * 2 + rows * c.K // 2 + rows * 4 * (1 if group == 0 else c.K // group)
        xs = copies(lambda: x.clone(), rows * c.K * 2)
        outs = [qr.rotate_quant(xx, rot, group) for xx in xs]
        ms = med(lambda i: qr.rotate_quant(xs[i % len(xs)], rot, group, *outs[i % len(xs)]), reps)
        emit(name, kernel="qr_rotate_quant", shape=[rows, c.K], group=group, us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, buffers=len(xs))

    def gemm_case(name, M, N, K, group, reps=20, single=False):
        if only and name not in only:
            return
        G = 1 if group == 0 else K // group
        wbytes = N * K // 2 + N * G * 4
        nw = 1 if single else max(2, -(-CACHE_BYTES // wbytes))
        a = codes(M, K)
        sa = torch.rand((M,) if group == 0 else (M, G), device=dev, generator=g) * 0.01
        ws = [codes(N, K) for _ in range(nw)]
        sw = torch.rand((N,) if group == 0 else (N, G), device=dev, generator=g) * 0.01
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ms = med(lambda i: qr.int4_gemm(a, sa, ws[i % nw], sw, group, y=y), reps)
        ops = 2.0 * M * N * K
        nbytes = M * K // 2 + N * K // 2 + M * N * 2 + 4 * G * (M + N)
        emit(name, kernel="qr_int4_gemm", shape=[M, N, K], group=group, us=round(ms * 1e3, 3),
             TOPS=round(ops / ms / 1e9, 2), frac_int8=round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, weight_sets=nw, **({"mode": "single-shot latency (weights cached)"} if single else {}))

    def gemm8_case(name, M, N, K, group, reps=20):
        if only and name not in only:
            return
        G = 1 if group == 0 else K // group
        nw = max(2, -(-CACHE_BYTES // (N * K)))
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        ws = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g) for _ in range(nw)]
        sa = torch.rand((M,) if group == 0 else (M, G), device=dev, generator=g) * 0.001
        sw = torch.rand((N,) if group == 0 else (N, G), device=dev, generator=g) * 0.001
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ms = med(lambda i: qr.int8_gemm(a, sa, ws[i % nw], sw, group, y=y), reps)
        ops = 2.0 * M * N * K
        emit(name, kernel="qr_int8_gemm", shape=[M, N, K], group=group, us=round(ms * 1e3, 3),
             TOPS=round(ops / ms / 1e9, 2), frac_int8=round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4), weight_sets=nw)

    def rq8_case(name, cfg, rows, group, bits, reps=20):
        if only and name not in only:
            return
        c = W.CONFIGS[cfg]
        x = torch.from_numpy(W.make_x(c, rows=np.arange(rows))).to(dev)
        rot = qr.Rotation.hadamard(c.K, W.make_signs(c))
        nbytes = rows * c.K * 2 + rows * c.K + rows * 4 * (1 if group == 0 else c.K // group)
        xs = copies(lambda: x.clone(), rows * c.K * 2)
        outs = [qr.rotate_quant_i8(xx, rot, bits, group) for xx in xs]
        ms = med(lambda i: qr.rotate_quant_i8(xs[i % len(xs)], rot, bits, group, *outs[i % len(xs)]), reps)
        emit(name, kernel="qr_rotate_quant_i8", shape=[rows, c.K], bits=bits, group=group, us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, buffers=len(xs))

    def swiglu_case(name, cfg, rows, reps=20):
        if only and name not in only:
            return
        c = W.CONFIGS[cfg]
        gus = copies(lambda: torch.randn((rows, 2 * c.K), device=dev, generator=g).half(), rows * c.K * 4)
        rot = qr.Rotation.kronecker(c.had_n, W.make_dense(c), W.make_signs(c))
        out = qr.swiglu_rotate_quant(gus[0][:, :c.K], gus[0][:, c.K:], rot)
        ms = med(lambda i: qr.swiglu_rotate_quant(gus[i % len(gus)][:, :c.K], gus[i % len(gus)][:, c.K:], rot, 0,
                                                  *out), reps)
        nbytes = rows * c.K * 4 + rows * c.K // 2 + rows * 4
        emit(name, kernel="qr_swiglu_rotate_quant", shape=[rows, c.K], us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), bytes=nbytes,
             buffers=len(gus))

    def kv_case(name, T, reps=20, single=False):
        if only and name not in only:
            return
        H = 32
        if T <= 64:
            k, _ = W.make_kv("c5")
        else:
            k = W.make_kv_large(T, H)
        kt = torch.from_numpy(k).to(dev)
        nbytes = T * H * (256 + 64 + 5)
        ks = [kt] if single else copies(lambda: kt.clone(), T * H * 256)
        outs = [qr.kv_quant(kk) for kk in ks]
        ms = med(lambda i: qr.kv_quant(ks[i % len(ks)], None, *outs[i % len(ks)]), reps)
        emit(name, kernel="qr_kv_quant", shape=[T, H, 128], us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, buffers=len(ks), **({"mode": "single-shot latency"} if single else {}))

    def attn_case(name, B, T, Hq, Hkv, reps=20):
        if only and name not in only:
            return
        per = 2 * B * T * Hkv * 69
        nsets = max(2, -(-CACHE_BYTES // per))

        def make():
            return (torch.randint(0, 256, (B, T, Hkv, 64), dtype=torch.uint8, device=dev, generator=g),
                    torch.rand((B, T, Hkv), device=dev, generator=g) * 0.28 + 0.02,
                    torch.randint(0, 16, (B, T, Hkv), dtype=torch.uint8, device=dev, generator=g),
                    torch.randint(0, 256, (B, T, Hkv, 64), dtype=torch.uint8, device=dev, generator=g),
                    torch.rand((B, T, Hkv), device=dev, generator=g) * 0.28 + 0.02,
                    torch.randint(0, 16, (B, T, Hkv), dtype=torch.uint8, device=dev, generator=g))
        caches = [make() for _ in range(nsets)]
        q = torch.randn((B, Hq, 128), device=dev, generator=g).half()
        out = torch.empty_like(q)
        wsb = qr.kv_attn_decode_workspace(B, Hq, Hkv, T)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev)
        nbytes = B * T * Hkv * (2 * 64 + 2 * 5) + 2 * B * Hq * 128 * 2
        ms = med(lambda i: qr.kv_attn_decode(q, *caches[i % nsets], out=out, workspace=ws), reps)
        emit(name, kernel="qr_kv_attn_decode", shape=[B, T, Hq, Hkv], us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, workspace=wsb, cache_sets=nsets)

    if not only or "peaks" in only:
        pk = measure_peaks(dev)
        # the suite's GEMM cases multiply uniformly random codes: the same
        # MFMA loop on such codes is their data-matched ceiling
        ra, rw = codes(4096, 32768), codes(4096, 32768)
        pk["mfma_int8_random_codes_TOPS"] = measure_codes_peak(ra, rw, st)
        del ra, rw
        emit("peaks", **pk)
    rq_case("rq_c2", "c2", 2048, 0)
    rq_case("rq_c4_g128", "c4", 16384, 128)
    rq_case("rq_c5", "c5", 64, 0)
    rq_case("rq_c3_kron", "c3", 131072, 0)
    rq_case("rq_d70_kron", "d70", 16384, 0)
    gemm_case("gemm_c2", 2048, 12288, 4096, 0)
    gemm_case("gemm_c3", 131072, 4096, 11008, 0)
    gemm_case("gemm_c4_g128", 16384, 28672, 8192, 128)
    gemm_case("gemm_c5_decode_single", 64, 4096, 4096, 0, reps=50, single=True)
    gemm_case("gemm_c5_decode_streamed", 64, 4096, 4096, 0, reps=128)
    kv_case("kv_c5_decode", 64, reps=50, single=True)
    kv_case("kv_prefill_131072", 131072)
    swiglu_case("swiglu_rq_d70", "d70", 16384)
    gemm8_case("gemm8_c2", 2048, 12288, 4096, 0)
    gemm8_case("gemm8_c4_g128", 16384, 28672, 8192, 128)
    gemm8_case("gemm8_c5_decode", 64, 4096, 4096, 0, reps=50)
    rq8_case("rq8_c2", "c2", 2048, 0, 8)
    rq8_case("rq8_c4_g128", "c4", 16384, 128, 8)
    attn_case("attn_decode_b64_t2048", 64, 2048, 32, 32)
    attn_case("attn_decode_b1_t4096", 1, 4096, 32, 32, reps=50)
    attn_case("attn_decode_gqa_b64_t2048", 64, 2048, 64, 8)


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_last)
        return
    if args.ingest_pmc:
        ingest_pmc(args.config, args.ingest_pmc[0], args.ingest_pmc[1], args.calib_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the hot path is per-token independent and would shard tokens across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    if args.codes_sweep:
        codes_sweep(args)
        return
    if args.suite:
        import torch
        import rotation_bit_quantized_amd as qr
        qr.library()
        torch.cuda.set_device(0)
        suite(args)
        return
    run_step(args)


if __name__ == "__main__":
    main()
