#!/usr/bin/env python3
"""Throughput of QuaRot's 4-bit linear-layer hot path on one MI355X.

One step = one pass of the whole path over one batch, in order on one HIP
stream:
  qr_rotate_quant  x [M, K] fp16 -> int4 codes + per-token scales
  qr_int4_gemm     codes x pre-rotated int4 weights -> y [M, N] fp16
  qr_kv_quant      the K and V slices of y (fused QKV output), 32 heads x 128
Consecutive steps (independent batches) alternate over --streams HIP streams
of default priority, so that one batch's small, latency-bound kernels run
beside another batch's GEMM; a buffer set is reused only after the step that
last used it has finished (an event dependency).
Default workload: LLaMA-2-7B fused QKV prefill, x 2048 x 4096 -> 12288 (the
layer the QuaRot summary's prefill figures are about: batch 64 x 2048 tokens
in one block).  Inputs are synthetic and seeded (package ``workloads``);
weights are prepared on the GPU before timing (rotate + quantize the rows of
W^T with the same library call).  To keep the measurement honest about HBM,
steps cycle through enough distinct buffer sets (>= 1 GiB) that nothing is
served from the 256 MB Infinity Cache between uses.

Prints one JSON line.  `value` is whole-step throughput in TOPS (2 M N K per
step).  `roofline` is for the dominant kernel (the int4 GEMM) with its
average launch time from HIP events recorded around each launch on the
launch stream.  `cpu_baseline` is the CPU oracle timed on a bounded row
sample of the same workload.

  python bench.py [--steps 20] [--warmup 5] [--config c2] [--streams 2] [--no-cpu]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, published (5.0 POP/s)
CACHE_BYTES = 1 << 30        # cycle buffers over >= 1 GiB (MALL is 256 MB)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", choices=["c2"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cpu-rows", type=int, default=0, help="token rows in the CPU oracle sample (0 = all)")
    ap.add_argument("--streams", type=int, default=2,
                    help="HIP streams the steps alternate over (1: strictly one step after another)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    ap.add_argument("--sets", type=int, default=0, help="buffer sets to cycle (0 = enough for 1 GiB)")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the step, time each kernel at every config's shape (one JSON line each)")
    ap.add_argument("--only", default="", help="with --suite: comma-separated case names to run")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="read rocprofv3 FETCH_SIZE / WRITE_SIZE runs of `bench.py --copy-calib MIB` and write "
                         "profiles/traffic.json (HBM bytes per launch of the GEMM, copy-calibrated)")
    ap.add_argument("--calib-mib", type=int, default=1024, help="size of the copy used with --ingest-pmc")
    return ap.parse_args()


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key, src_files, launches_bytes):
    """HBM bytes of one launch from committed rocprofv3 counter runs, or None
    when they are missing or the kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[kernel_key]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_hash") != source_hash(src_files):
        return None
    return {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
            "total_bytes": rec["fetch_bytes"] + rec["write_bytes"], "algorithmic_bytes": launches_bytes,
            "calibration": rec.get("calibration")}


def cpu_baseline(cfg, rows):
    """The oracle on a bounded sample: `rows` token rows through rotate,
    quantize, int64 GEMM against all N output channels, dequantize and the KV
    quantizer on those rows' K and V slices.  Weight preparation (offline in
    the method) is not timed."""
    import oracle as O
    import workloads as W
    threads = len(os.sched_getaffinity(0))
    x = W.make_x(cfg, rows=np.arange(rows))
    w = W.make_w(cfg)
    r = O.rotation_matrix(cfg.K, signs=W.make_signs(cfg))
    qw, sw = O.quantize_weights(O.rotate_weights(w, r), cfg.group)
    t0 = time.perf_counter()
    y = O.rotate(x, r)
    qx, sx, _ = O.quantize_symmetric(y, cfg.group)
    blocks = np.array_split(np.arange(cfg.N), threads)
    with cf.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda b: O.int_gemm(qx, qw[b], cfg.group), blocks))
    acc = np.concatenate(parts, axis=-1)
    out = O.dequantize_output(acc, sx, sw, cfg.group)
    hq = cfg.K  # K and V slices of the fused output: heads of 128
    kv = out.astype(np.float16)
    O.kv_quantize(kv[:, hq:2 * hq].reshape(rows, hq // 128, 128))
    O.kv_quantize(kv[:, 2 * hq:3 * hq].reshape(rows, hq // 128, 128))
    dt = time.perf_counter() - t0
    ops = 2.0 * rows * cfg.N * cfg.K
    return {"value": round(ops / dt / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{rows} of {cfg.M} token rows: fp64 explicit-matrix rotation, RTN, int64 GEMM against "
                      f"all {cfg.N} channels (column blocks over {threads} threads), fp64 dequant, KV quant of "
                      f"the sampled rows' K/V; weight prep untimed"}


GEMM_SOURCES = ["rotation_bit_quantized_amd/csrc/gemm_prefill.hip", "rotation_bit_quantized_amd/csrc/qr_common.h"]


def ingest_pmc(fetch_dir, write_dir, calib_mib):
    """Average FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the prefill GEMM
    and of the calibration copy; scale the GEMM's by known/measured of the
    copy (a copy of B bytes reads B and writes B)."""
    import csv
    import glob

    def per_dispatch(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] == counter:
                    key = (row["Dispatch_Id"], row["Kernel_Name"])
                    vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        return vals

    def gemm_avg(vals):
        v = [x for (d, k), x in vals.items() if "gemm_prefill_kernel" in k]
        if not v:
            raise SystemExit("no GEMM dispatches in the counter data")
        return sum(v) / len(v), [k for (d, k) in vals if "gemm_prefill_kernel" in k][0]

    def copy_max(vals):
        v = [x for (d, k), x in vals.items() if "copy" in k.lower()]
        if not v:
            raise SystemExit("no copy dispatch in the counter data")
        return max(v)

    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    g_fetch, gname = gemm_avg(fetch)
    g_write, _ = gemm_avg(write)
    known_kib = calib_mib * 1024.0
    f_scale = known_kib / copy_max(fetch)
    w_scale = known_kib / copy_max(write)
    import re
    m = re.search(r"gemm_prefill_kernel<[^>]*>", gname)
    rec = {"int4_gemm_c2": {
        "kernel": m.group(0) if m else gname[:80], "source_hash": source_hash(GEMM_SOURCES),
        "fetch_bytes": round(g_fetch * 1024 * f_scale), "write_bytes": round(g_write * 1024 * w_scale),
        "calibration": {"copy": f"device copy of {calib_mib} MiB (largest copy dispatch)",
                        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
                        "raw_fetch_kib": round(g_fetch, 1), "raw_write_kib": round(g_write, 1)},
        "command": "rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- python3 bench.py "
                   f"--steps 3 --warmup 1 --no-cpu --copy-calib {calib_mib}"}}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(rec))


def time_launches(fn, n, warm=3):
    """Average duration (ms) of fn(i) over n launches, HIP events on the
    current stream around the whole sequence."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n


def time_each(fn, n, stream, warm=3):
    """Average duration (ms) of one launch of fn(i): a HIP event pair on the
    launch stream around each of n launches (the per-dispatch span, as a
    kernel trace reports it; gaps between launches are not counted)."""
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
    return sum(a.elapsed_time(b) for a, b in ev) / n


def suite(args):
    """Kernel-level throughput at each config's shape.  Buffers are cycled so
    the data touched per launch comes from HBM, not the 256 MB cache, unless
    the case is explicitly a latency (single-shot) case."""
    import torch
    import workloads as W
    import rotation_bit_quantized_amd as qr
    dev = torch.device("cuda:0")
    only = set(filter(None, args.only.split(",")))
    g = torch.Generator(device=dev)
    g.manual_seed(1234)

    def codes(rows, k):
        return torch.randint(0, 256, (rows, k // 2), dtype=torch.uint8, device=dev, generator=g)

    def emit(case, **kw):
        print(json.dumps({"case": case, **kw}), flush=True)

    def copies(make, per_bytes):
        n = max(1, -(-CACHE_BYTES // max(1, per_bytes)))
        return [make() for _ in range(n)]

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
        ms = time_launches(lambda i: qr.rotate_quant(xs[i % len(xs)], rot, group, *outs[i % len(xs)]), reps)
        emit(name, kernel="qr_rotate_quant", shape=[rows, c.K], group=group, us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, buffers=len(xs))

    def gemm_case(name, M, N, K, group, reps=10, stream_w=1):
        if only and name not in only:
            return
        G = 1 if group == 0 else K // group
        a = codes(M, K)
        sa = torch.rand((M,) if group == 0 else (M, G), device=dev, generator=g) * 0.01
        ws = [codes(N, K) for _ in range(stream_w)]
        sw = torch.rand((N,) if group == 0 else (N, G), device=dev, generator=g) * 0.01
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ms = time_launches(lambda i: qr.int4_gemm(a, sa, ws[i % stream_w], sw, group, y=y), reps)
        ops = 2.0 * M * N * K
        nbytes = M * K // 2 + N * K // 2 + M * N * 2 + 4 * G * (M + N)
        emit(name, kernel="qr_int4_gemm", shape=[M, N, K], group=group, us=round(ms * 1e3, 3),
             TOPS=round(ops / ms / 1e9, 2), frac_int8=round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, weight_sets=stream_w)

    def gemm8_case(name, M, N, K, group, reps=10):
        if only and name not in only:
            return
        G = 1 if group == 0 else K // group
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        w = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
        sa = torch.rand((M,) if group == 0 else (M, G), device=dev, generator=g) * 0.001
        sw = torch.rand((N,) if group == 0 else (N, G), device=dev, generator=g) * 0.001
        y = torch.empty((M, N), dtype=torch.float16, device=dev)
        ms = time_launches(lambda i: qr.int8_gemm(a, sa, w, sw, group, y=y), reps)
        ops = 2.0 * M * N * K
        emit(name, kernel="qr_int8_gemm", shape=[M, N, K], group=group, us=round(ms * 1e3, 3),
             TOPS=round(ops / ms / 1e9, 2), frac_int8=round(ops / ms / 1e9 / INT8_PEAK_TOPS, 4))

    def rq8_case(name, cfg, rows, group, bits, reps=20):
        if only and name not in only:
            return
        c = W.CONFIGS[cfg]
        x = torch.from_numpy(W.make_x(c, rows=np.arange(rows))).to(dev)
        rot = qr.Rotation.hadamard(c.K, W.make_signs(c))
        nbytes = rows * c.K * 2 + rows * c.K + rows * 4 * (1 if group == 0 else c.K // group)
        xs = copies(lambda: x.clone(), rows * c.K * 2)
        outs = [qr.rotate_quant_i8(xx, rot, bits, group) for xx in xs]
        ms = time_launches(lambda i: qr.rotate_quant_i8(xs[i % len(xs)], rot, bits, group, *outs[i % len(xs)]),
                           reps)
        emit(name, kernel="qr_rotate_quant_i8", shape=[rows, c.K], bits=bits, group=group, us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, buffers=len(xs))

    def swiglu_case(name, cfg, rows, reps=3):
        if only and name not in only:
            return
        c = W.CONFIGS[cfg]
        gu = torch.randn((rows, 2 * c.K), device=dev, generator=g).half()   # fused gate/up output [rows, 2n]
        rot = qr.Rotation.kronecker(c.had_n, W.make_dense(c), W.make_signs(c))
        out = qr.swiglu_rotate_quant(gu[:, :c.K], gu[:, c.K:], rot)
        ms = time_each(lambda i: qr.swiglu_rotate_quant(gu[:, :c.K], gu[:, c.K:], rot, 0, *out), reps,
                       torch.cuda.current_stream())
        nbytes = rows * c.K * 4 + rows * c.K // 2 + rows * 4
        emit(name, kernel="qr_swiglu_rotate_quant", shape=[rows, c.K], us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4), bytes=nbytes)

    def kv_case(name, T, reps=20, cycle=True):
        if only and name not in only:
            return
        H = 32
        if T <= 64:
            k, _ = W.make_kv("c5")
        else:
            k = W.make_kv_large(T, H)
        kt = torch.from_numpy(k).to(dev)
        nbytes = T * H * (256 + 64 + 5)
        ks = copies(lambda: kt.clone(), T * H * 256) if cycle else [kt]
        outs = [qr.kv_quant(kk) for kk in ks]
        ms = time_launches(lambda i: qr.kv_quant(ks[i % len(ks)], None, *outs[i % len(ks)]), reps)
        emit(name, kernel="qr_kv_quant", shape=[T, H, 128], us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, buffers=len(ks))

    def attn_case(name, B, T, Hq, Hkv, reps=20):
        if only and name not in only:
            return
        kc = torch.randint(0, 256, (B, T, Hkv, 64), dtype=torch.uint8, device=dev, generator=g)
        vc = torch.randint(0, 256, (B, T, Hkv, 64), dtype=torch.uint8, device=dev, generator=g)
        ks = torch.rand((B, T, Hkv), device=dev, generator=g) * 0.28 + 0.02
        vs = torch.rand((B, T, Hkv), device=dev, generator=g) * 0.28 + 0.02
        kz = torch.randint(0, 16, (B, T, Hkv), dtype=torch.uint8, device=dev, generator=g)
        vz = torch.randint(0, 16, (B, T, Hkv), dtype=torch.uint8, device=dev, generator=g)
        q = torch.randn((B, Hq, 128), device=dev, generator=g).half()
        out = torch.empty_like(q)
        wsb = qr.kv_attn_decode_workspace(B, Hq, Hkv, T)
        ws = torch.empty((max(wsb, 16),), dtype=torch.uint8, device=dev)
        nbytes = B * T * Hkv * (2 * 64 + 2 * 5) + 2 * B * Hq * 128 * 2
        ms = time_each(lambda i: qr.kv_attn_decode(q, kc, ks, kz, vc, vs, vz, out=out, workspace=ws), reps,
                       torch.cuda.current_stream())
        emit(name, kernel="qr_kv_attn_decode", shape=[B, T, Hq, Hkv], us=round(ms * 1e3, 3),
             GBs=round(nbytes / ms / 1e6, 1), frac_hbm=round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
             bytes=nbytes, workspace=wsb)

    rq_case("rq_c2", "c2", 2048, 0)
    rq_case("rq_c4_g128", "c4", 16384, 128)
    rq_case("rq_c5", "c5", 64, 0)
    rq_case("rq_c3_kron", "c3", 16384, 0, reps=5)
    rq_case("rq_d70_kron", "d70", 16384, 0, reps=3)
    gemm_case("gemm_c2", 2048, 12288, 4096, 0)
    gemm_case("gemm_c3", 131072, 4096, 11008, 0, reps=3)
    gemm_case("gemm_c4_g128", 16384, 28672, 8192, 128, reps=3)
    gemm_case("gemm_c5_decode_single", 64, 4096, 4096, 0, reps=50)
    gemm_case("gemm_c5_decode_streamed", 64, 4096, 4096, 0, reps=128, stream_w=64)
    kv_case("kv_c5_decode", 64, reps=50, cycle=False)
    kv_case("kv_prefill_131072", 131072, reps=5)
    swiglu_case("swiglu_rq_d70", "d70", 16384)
    gemm8_case("gemm8_c2", 2048, 12288, 4096, 0)
    gemm8_case("gemm8_c4_g128", 16384, 28672, 8192, 128, reps=3)
    gemm8_case("gemm8_c5_decode", 64, 4096, 4096, 0, reps=50)
    rq8_case("rq8_c2", "c2", 2048, 0, 8)
    rq8_case("rq8_c4_g128", "c4", 16384, 128, 8)
    attn_case("attn_decode_b64_t2048", 64, 2048, 32, 32)
    attn_case("attn_decode_b1_t4096", 1, 4096, 32, 32, reps=50)
    attn_case("attn_decode_gqa_b64_t2048", 64, 2048, 64, 8)


def main():
    args = parse()
    if args.ingest_pmc:
        ingest_pmc(args.ingest_pmc[0], args.ingest_pmc[1], args.calib_mib)
        return
    if args.suite:
        import torch
        import rotation_bit_quantized_amd as qr
        qr.library()
        torch.cuda.set_device(0)
        suite(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the hot path is per-token independent and would shard tokens across GPUs with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import rotation_bit_quantized_amd as qr

    qr.library()                     # no fallback: fail loudly without the HIP library
    cfg = W.CONFIGS[args.config]
    M, N, K = cfg.M, cfg.N, cfg.K
    H = K // 128
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---------------------------------------------------------- resident inputs (untimed)
    x_host = W.make_x(cfg)
    w_host = W.make_w(cfg)
    rot = qr.Rotation.hadamard(K, W.make_signs(cfg))
    x0 = torch.from_numpy(x_host).to(dev)
    wt = torch.from_numpy(np.ascontiguousarray(w_host.T)).to(dev)
    wc0, ws0 = qr.rotate_quant(wt, rot, cfg.group)          # offline weight prep, on the GPU
    del wt
    set_bytes = (x0.numel() * 2 + M * K // 2 + M * 4 + wc0.numel() + ws0.numel() * 4 + M * N * 2
                 + 2 * (M * H * 64 + M * H * 5))
    nsets = args.sets or max(1, -(-CACHE_BYTES // set_bytes))
    sets = []
    for i in range(nsets):
        s = dict(x=x0.clone(), wc=wc0.clone(), ws=ws0.clone(),
                 xc=torch.empty((M, K // 2), dtype=torch.uint8, device=dev),
                 xs=torch.empty((M,), dtype=torch.float32, device=dev),
                 y=torch.empty((M, N), dtype=torch.float16, device=dev),
                 # the K and V heads of a token side by side: [M][2H] vectors
                 kvc=torch.empty((M, 2 * H, 64), dtype=torch.uint8, device=dev),
                 kvs=torch.empty((M, 2 * H), dtype=torch.float32, device=dev),
                 kvz=torch.empty((M, 2 * H), dtype=torch.uint8, device=dev))
        sets.append(s)
    del x0, wc0, ws0
    stream = torch.cuda.current_stream()
    # default-priority streams only
    streams = [stream] + [torch.cuda.Stream(device=dev) for _ in range(max(1, args.streams) - 1)]

    def rq(s, st=stream):
        qr.rotate_quant(s["x"], rot, cfg.group, codes=s["xc"], scales=s["xs"], stream=st)

    def gemm(s, st=stream):
        qr.int4_gemm(s["xc"], s["xs"], s["wc"], s["ws"], cfg.group, y=s["y"], stream=st)

    def kv(s, st=stream):
        # K and V are adjacent column ranges of the QKV output: one launch
        # quantizes the 2H head vectors of every token
        qr.kv_quant(s["y"][:, K:3 * K], codes=s["kvc"], scales=s["kvs"], zeros=s["kvz"], stream=st)

    def step(i):
        s = sets[i % nsets]
        st = streams[i % len(streams)]
        if "done" in s and s["done_on"] is not st:
            st.wait_event(s["done"])   # the set's previous step, on another stream, has finished
        rq(s, st)
        gemm(s, st)
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

    if args.copy_calib:
        nb = args.copy_calib << 20
        a = torch.empty(nb, dtype=torch.uint8, device=dev)
        b = torch.empty(nb, dtype=torch.uint8, device=dev)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    fork()
    for i in range(args.warmup):
        step(i)
    join()
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps, nothing else on the stream
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
    gpu_ms = start.elapsed_time(end)
    ms_per_step = gpu_ms / args.steps

    # per-kernel durations (after the timed region, same stream, the rotating
    # buffer sets): a HIP event pair around each launch
    nrep = max(10, args.steps)
    rq_ms = time_each(lambda i: rq(sets[i % nsets]), nrep, stream)
    gemm_ms = time_each(lambda i: gemm(sets[i % nsets]), nrep, stream)
    kv_ms = time_each(lambda i: kv(sets[i % nsets]), nrep, stream)

    ops = 2.0 * M * N * K
    value = ops / (ms_per_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_ms * 1e-3) / 1e12
    rq_bytes = M * K * 2 + M * K // 2 + M * 4
    kv_bytes = 2 * (M * H * 128 * 2 + M * H * 64 + M * H * 5)
    gemm_bytes = M * K // 2 + N * K // 2 + M * 4 + N * 4 + M * N * 2
    traffic = load_traffic("int4_gemm_c2", GEMM_SOURCES, gemm_bytes)

    out = {
        "metric": "rotate+quant+int4 GEMM TOPS and GB/s at 7B/70B layer shapes; % of roofline",
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
            "workload": f"{cfg.name}: {cfg.desc}; rotate D.H_{K} + per-token int4 RTN, int4 GEMM (int8 MFMA, "
                        f"per-channel int4 weights, fp16 out), 4-bit KV quant of the K and V heads (one launch, {M}x{2 * H}x128)",
            "M": M, "N": N, "K": K, "group": cfg.group, "codes": "int4", "mfma": "int8 -> int32",
            "rotation": "fp32 (fp16-MFMA first factor)", "buffer_sets": nsets, "streams": len(streams),
        },
        "kernels": {
            "rotate_quant": {"us": round(rq_ms * 1e3, 3), "GB/s": round(rq_bytes / (rq_ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(rq_bytes / (rq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                             "bytes": rq_bytes},
            "int4_gemm": {"us": round(gemm_ms * 1e3, 3), "TOPS": round(gemm_tops, 2),
                          "frac_int8_peak": round(gemm_tops / INT8_PEAK_TOPS, 4), "bytes": gemm_bytes},
            "kv_quant_KV": {"us": round(kv_ms * 1e3, 3), "GB/s": round(kv_bytes / (kv_ms * 1e-3) / 1e9, 1),
                            "frac_hbm": round(kv_bytes / (kv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "bytes": kv_bytes},
        },
        "roofline": {
            "bound": "mfma", "kernel": "int4_gemm (gemm_prefill_kernel)",
            "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
            "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
            "traffic": None if traffic is None else traffic["total_bytes"],
            "traffic_detail": traffic,
        },
        "wall_s": round(wall, 4),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, min(args.cpu_rows or M, M))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
