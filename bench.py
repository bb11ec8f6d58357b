#!/usr/bin/env python3
"""Throughput of exact tiled attention on one MI355X, fwd and fwd+bwd.

One step = one pass of the whole path over one batch of synthetic input:
the forward kernel (O, L), then the backward stages (query-outer dQ kernel,
which also forms the row terms D and L * log2(e), then the key-outer dK/dV
kernel).  The default workload is the
headline one: B=2, H=32, N=4096, d=128, bf16, causal.

    python bench.py [--steps K] [--warmup W] [--workload c3]
                    [--no-cpu-baseline] [--gpus 1]

Prints one JSON line.  Work is counted as 4 N^2 d per head forward and
10 N^2 d backward (five contractions), halved when causal.  Of the five
backward contractions the dK/dV kernel performs four (S, dP, dV, dK) and the
dQ kernel one (dQ); the dQ kernel's second evaluation of S and dP is extra
work of the split and is reported separately, not counted.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402
from workloads import cost  # noqa: E402

METRIC = ("attention TFLOP/s fwd & fwd+bwd, N=4096 d=128 causal bf16; "
          "% MFMA peak")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
PEAK_FP32_VALU_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c3",
                    choices=sorted(W.WORKLOADS) + sorted(W.KV_WORKLOADS)
                    + ["varlen", "fp8", "drop", "pad"],
                    help="an attention workload (c1..c5), a split-KV "
                         "decode workload (dec), a packed batch of "
                         "mixed-length sequences (varlen), the FP8 "
                         "forward on the headline shape (fp8), fwd+bwd "
                         "with dropout on the headline shape (drop), or "
                         "fwd+bwd with key padding at B=64 H=16 N=1024 "
                         "d=64 (pad)")
    ap.add_argument("--splits", type=int, default=0,
                    help="split count for a decode workload (0: its own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="the oracle's timed sample stops after the first "
                         "head that brings its wall time past this")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="measure the dense bf16 and fp8 matrix-core peak "
                         "and the shader clock (libfa355_probe.so)")
    ap.add_argument("--atomic-probe", action="store_true",
                    help="time the fp32 atomic traffic of a dQ formed inside "
                         "the dK/dV kernel at the headline shape "
                         "(libfa355_probe.so) and exit")
    ap.add_argument("--coexec-probe", action="store_true",
                    help="measure how MFMA, VALU, exp and LDS reads share a "
                         "CU (libfa355_probe.so) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="time fwd and bwd over sequence lengths 256..16384 "
                         "at 16384 tokens per batch (B = 16384 / N), H=32, "
                         "d 64 and 128, dense and causal; one JSON line per "
                         "point, then exit")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three "
                         "times (calibrates the HBM byte counters) and exit")
    ap.add_argument("--traffic-json", default=os.path.join(
        ROOT, "profiles", "traffic.json"),
        help="per-dispatch HBM bytes measured with rocprofv3 counters")
    return ap.parse_args()


def source_digest() -> str:
    """Digest of the HIP sources the measured attention library was built
    from (the measurement-aid probe library's sources excluded)."""
    import hashlib
    from io_aware_exact_04_amd import build as B
    csrc = os.path.join(ROOT, "io_aware_exact_04_amd", "csrc")
    probe = set(B.PROBE_SOURCES) | {"fa355_probe.map"}
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f in probe:
            continue
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def shader_clock_mhz():
    """The shader clock at this moment, under matrix-core load: one short
    launch of the probe library's MFMA kernel (about half a millisecond),
    whose first wave reads the shader-clock counter (s_memtime) against the
    100 MHz reference counter (s_memrealtime).  None if the probe library
    is not built."""
    import ctypes
    import torch
    from io_aware_exact_04_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        return None
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.fa355_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.fa355_mfma_probe.restype = ctypes.c_int
    blocks = 512
    clocks = torch.zeros(4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    rc = lib.fa355_mfma_probe(0, 2000, blocks, clocks.data_ptr(),
                              sink.data_ptr(), stream.cuda_stream)
    torch.cuda.synchronize()
    if rc != 0:
        return None
    c = clocks.cpu().tolist()
    return round(100.0 * (c[1] - c[0]) / max(c[3] - c[2], 1))


def spread(xs):
    """Median, 10th and 90th percentile of a list of times."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def describe(w):
    s = (f"{w.name}: B={w.B} H={w.H} N={w.N} d={w.D} {w.dtype}"
         f"{' causal' if w.causal else ''}")
    if w.has_mask:
        s += f" block-mask {w.mask_block} (band {w.mask_band} + "
        s += f"{w.mask_frac:.0%} random)"
    if w.k_scale != 1.0:
        s += f" K x{w.k_scale:g}"
    return s


def cpu_baseline(w, inp, min_seconds: float):
    """The fp64 oracle as it stands, timed on the host on a bounded sample:
    whole heads, forward then backward, until ``min_seconds`` have passed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?")
                                for p in threadpool_info()
                                if p.get("user_api") == "blas"}))
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads, blas = os.cpu_count() or 1, "unknown"
    mb = w.mask_block or 128
    hs = []
    t0 = time.perf_counter()
    for b, h in ((b, h) for b in range(w.B) for h in range(w.H)):
        oracle.forward_head(inp["q"][b, h], inp["k"][b, h], inp["v"][b, h],
                            w.scale, w.causal, inp["block_mask"], mb)
        if w.backward:
            oracle.backward_head(inp["q"][b, h], inp["k"][b, h],
                                 inp["v"][b, h], inp["do"][b, h], w.scale,
                                 w.causal, inp["block_mask"], mb)
        hs.append((b, h))
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    flops = cost.fwd_flops(1, len(hs), w.N, w.D, w.causal, inp["block_mask"],
                           mb)
    if w.backward:
        flops += cost.bwd_flops(1, len(hs), w.N, w.D, w.causal,
                                inp["block_mask"], mb)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(threads), "kind": "oracle",
            "sample": (f"{len(hs)} of {w.B * w.H} heads of {w.name}, "
                       f"{'fwd+bwd' if w.backward else 'fwd'}, fp64 numpy "
                       f"({blas}), {dt:.1f} s wall; counted FLOPs of the "
                       f"sample / wall time (the oracle also evaluates "
                       f"masked entries)")}


def bench_decode(args):
    """Split-KV forward on a decode workload: HBM-bound (every key and value
    is read once), reported as GB/s of algorithmic bytes against 8 TB/s."""
    import torch
    import io_aware_exact_04_amd as fa
    w = W.KV_WORKLOADS[args.workload]
    splits = args.splits or w.num_splits
    inp = W.make_kv_inputs(w)
    q, k, v = (W.to_torch(inp[x], w.dtype, "cuda") for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(fa.splitkv_workspace_bytes(q, k, splits), 16),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        fa.fa_fwd_splitkv(q, k, v, w.scale, w.causal, splits, out=o, lse=lse,
                          workspace=ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    # Algorithmic bytes: Q, K, V read once, O and L written once.
    nbytes = (2 * w.B * w.H * (w.Nq + 2 * w.Nk) * w.D
              + 2 * w.B * w.H * w.Nq * w.D + 4 * w.B * w.H * w.Nq)
    gbs = nbytes / (us * 1e-6) / 1e9
    # Measured HBM bytes of one call (both kernels), if the counters were
    # taken on the current kernel sources.
    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f).get(w.name, {})
        if tj.get("source_sha256_16") == source_digest():
            traffic = tj.get("fwd_splitkv_call", {}).get("bytes_per_dispatch")
    except (OSError, ValueError):
        pass
    line = {
        "metric": "split-KV decode forward, GB/s of K/V streamed",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) inputs, see "
                                 "workloads.KV_WORKLOADS)",
        "config": {"workload": (f"{w.name}: B={w.B} H={w.H} Nq={w.Nq} "
                                f"Nk={w.Nk} d={w.D} bf16"
                                f"{' causal' if w.causal else ''}, "
                                f"{splits} splits")},
        "roofline": {"bound": "hbm", "kernel": "fwd_splitkv (partials + "
                     "merge, one call)", "achieved": round(gbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(us, 2),
                     "algorithmic_bytes_per_launch": nbytes},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_varlen(args):
    """Forward + backward of a packed batch of mixed-length causal sequences
    (16 sequences, lengths uniform on [256, 4096] from a fixed seed, H=32,
    d=128, bf16), against the same batch padded to the longest sequence
    through the [B, H, N, d] path.  Counted FLOPs are the useful ones
    (4 len^2 d forward, 10 len^2 d backward per head, halved for causal)."""
    import torch
    import io_aware_exact_04_amd as fa
    lengths = W.varlen_lengths(16, 256, 4096, seed=51)
    H, D = 32, 128
    inp = W.make_varlen_inputs(lengths, H, D, seed=52)
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    mx = max(lengths)
    B = len(lengths)
    qp, kp, vp, dop = (torch.zeros(B, H, mx, D, dtype=torch.bfloat16,
                                   device="cuda") for _ in range(4))
    for b, (a, e) in enumerate(zip(inp["cu_seqlens"][:-1],
                                   inp["cu_seqlens"][1:])):
        for src, dst in ((q, qp), (k, kp), (v, vp), (do, dop)):
            dst[b, :, : e - a] = src[a:e].permute(1, 0, 2)
    fl = sum((4 + 10) * n * n * D * H * 0.5 for n in lengths)

    def packed():
        o, lse = fa.fa_fwd_varlen(q, k, v, cu, mx, causal=True)
        fa.fa_bwd_varlen(q, k, v, o, lse, do, cu, mx, causal=True)

    def padded():
        o, lse = fa.fa_fwd(qp, kp, vp, causal=True)
        fa.fa_bwd(qp, kp, vp, o, lse, dop, causal=True)

    def time_it(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps
    t_pk = time_it(packed)
    t_pd = time_it(padded)
    line = {
        "metric": "packed varlen attention TFLOP/s, fwd+bwd (useful FLOPs)",
        "value": round(fl / t_pk / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_pk * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, seeded length mix)",
        "config": {"workload": (f"varlen: {B} causal sequences, lengths "
                                f"{min(lengths)}..{mx} (total "
                                f"{sum(lengths)}), H={H} d={D} bf16"),
                   "lengths": lengths},
        "padded_ms_per_step": round(t_pd * 1e3, 4),
        "padded_useful_tflops": round(fl / t_pd / 1e12, 2),
        "speedup_over_padded": round(t_pd / t_pk, 3),
        "roofline": {"bound": "mfma", "kernel": "fwd+bwd (all kernels)",
                     "achieved": round(fl / t_pk / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fl / t_pk / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_padding(args):
    """Forward + backward with a key-padding mask on the shape of the
    pages' key-padding experiment (batch 64, 16 heads, N = 1024, d = 64,
    bf16, no causal mask; valid keys per batch entry uniform on [256, 1024]),
    against the unpadded path on the same inputs.  Counted FLOPs cover the
    valid keys only; the compulsory HBM bytes are every input read once and
    every output written once (padded key rows neither read nor computed)."""
    import torch
    import io_aware_exact_04_amd as fa
    w = W.padding_workload()
    lens = W.padding_lengths(w.B, w.N)
    inp = W.make_inputs(w)
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    del inp
    kl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(fa.workspace_bytes(q), 16), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    Ev = torch.cuda.Event

    def padded(ev):
        ev[0].record(stream)
        fa.fa_fwd_ex(q, k, v, w.scale, False, 0.0, 0, kl, out=o, lse=lse)
        ev[1].record(stream)
        fa.fa_bwd_ex(q, k, v, o, lse, do, w.scale, False, 0.0, 0, kl,
                     workspace=ws, out=grads)
        ev[2].record(stream)

    def plain(ev):
        ev[0].record(stream)
        fa.fa_fwd(q, k, v, w.scale, False, out=o, lse=lse)
        ev[1].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, w.scale, False, workspace=ws,
                  out=grads)
        ev[2].record(stream)

    def run(fn):
        evs = [[Ev(enable_timing=True) for _ in range(3)]
               for _ in range(args.warmup + args.steps)]
        t0 = None
        for i, e in enumerate(evs):
            if i == args.warmup:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            fn(e)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        tail = evs[args.warmup:]
        f = float(np.mean([e[0].elapsed_time(e[1]) for e in tail]))
        b = float(np.mean([e[1].elapsed_time(e[2]) for e in tail]))
        return wall, f, b
    wall, f_ms, b_ms = run(padded)
    _, pf_ms, pb_ms = run(plain)
    valid = sum(lens)                       # valid keys over the batch
    fl_f = 4.0 * w.H * w.N * valid * w.D
    fl_b = 2.5 * fl_f
    e = 2 * w.H * w.D                       # bytes of one row of all heads
    qrows, krows = w.B * w.N, valid
    compulsory = ((qrows + 2 * krows) * e + qrows * e + 4 * w.B * w.H * w.N
                  + (2 * qrows + 2 * krows + qrows) * e + 4 * w.B * w.H * w.N
                  + qrows * e + 2 * w.B * w.N * e)
    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f).get("pad", {})
        if tj.get("source_sha256_16") == source_digest():
            traffic = tj.get("fwd_bwd_step", {}).get("bytes_per_step")
    except (OSError, ValueError):
        pass
    ach = (fl_f + fl_b) / ((f_ms + b_ms) * 1e-3) / 1e12
    line = {
        "metric": "attention TFLOP/s fwd+bwd with a key-padding mask, "
                  "B=64 H=16 N=1024 d=64 bf16",
        "value": round((fl_f + fl_b) / wall / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, valid keys per batch "
                "entry uniform on [256, 1024], see workloads)",
        "config": {"workload": "pad: B=64 H=16 N=1024 d=64 bf16, key "
                               f"padding ({valid} of {w.B * w.N} keys valid)"},
        "counted_gflop_fwd_bwd": round((fl_f + fl_b) / 1e9, 3),
        "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
        "unpadded_fwd_ms": round(pf_ms, 4), "unpadded_bwd_ms": round(pb_ms, 4),
        "compulsory_hbm_bytes": int(compulsory),
        "roofline": {"bound": "mfma", "kernel": "fwd+bwd (all kernels)",
                     "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_dropout(args):
    """Forward + backward with fused dropout (p = 0.1) on the headline shape
    (B=2, H=32, N=4096, d=128, causal, bf16), against the plain path on the
    same inputs.  Counted FLOPs as without dropout; the keep decisions
    (Philox4x32-10 per 4x4 block) are extra vector work in all three
    kernels."""
    import torch
    import io_aware_exact_04_amd as fa
    w = W.get("c3")
    inp = W.make_inputs(w)
    q, k, v, do = (W.to_torch(inp[x], "bf16", "cuda") for x in
                   ("q", "k", "v", "do"))
    p, seed = 0.1, 2024
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    grads = tuple(torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(fa.workspace_bytes(q), 16), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    Ev = torch.cuda.Event

    def drop(ev):
        ev[0].record(stream)
        fa.fa_fwd_ex(q, k, v, w.scale, True, p, seed, out=o, lse=lse)
        ev[1].record(stream)
        fa.fa_bwd_ex(q, k, v, o, lse, do, w.scale, True, p, seed,
                     workspace=ws, out=grads)
        ev[2].record(stream)

    def plain(ev):
        ev[0].record(stream)
        fa.fa_fwd(q, k, v, w.scale, True, out=o, lse=lse)
        ev[1].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, w.scale, True, workspace=ws,
                  out=grads)
        ev[2].record(stream)

    def run(fn):
        evs = [[Ev(enable_timing=True) for _ in range(3)]
               for _ in range(args.warmup + args.steps)]
        t0 = None
        for i, e in enumerate(evs):
            if i == args.warmup:
                torch.cuda.synchronize()
                t0 = time.perf_counter()
            fn(e)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        tail = evs[args.warmup:]
        f = float(np.mean([e[0].elapsed_time(e[1]) for e in tail]))
        b = float(np.mean([e[1].elapsed_time(e[2]) for e in tail]))
        return wall, f, b
    wall, f_ms, b_ms = run(drop)
    _, pf_ms, pb_ms = run(plain)
    fl_f = cost.fwd_flops(w.B, w.H, w.N, w.D, True, None, 128)
    fl_b = cost.bwd_flops(w.B, w.H, w.N, w.D, True, None, 128)
    line = {
        "metric": "attention TFLOP/s fwd+bwd with fused dropout p=0.1, "
                  "N=4096 d=128 causal bf16",
        "value": round((fl_f + fl_b) / wall / 1e12, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, see workloads)",
        "config": {"workload": "drop: " + describe(w) + ", dropout 0.1 "
                   "(Philox4x32-10, seed 2024)"},
        "fwd_ms": round(f_ms, 4), "bwd_ms": round(b_ms, 4),
        "plain_fwd_ms": round(pf_ms, 4), "plain_bwd_ms": round(pb_ms, 4),
        "dropout_overhead": round((f_ms + b_ms) / (pf_ms + pb_ms), 3),
        "roofline": {"bound": "mfma", "kernel": "fwd+bwd (all kernels)",
                     "achieved": round((fl_f + fl_b) / ((f_ms + b_ms) * 1e-3)
                                       / 1e12, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round((fl_f + fl_b) / ((f_ms + b_ms) * 1e-3)
                                   / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    print(json.dumps(line), flush=True)
    return 0


def mfma_probe():
    """Dense MFMA throughput and shader clock, measured: every wave of 2048
    workgroups x 4 waves runs 8 independent accumulation chains (bf16
    32x32x16, then fp8 32x32x64 with unit E8M0 scales); best of 5 launches
    timed with HIP events on the launch stream."""
    import ctypes
    import torch
    from io_aware_exact_04_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.fa355_mfma_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    lib.fa355_mfma_probe.restype = ctypes.c_int
    blocks = 2048
    clocks = torch.zeros(4, dtype=torch.int64, device="cuda")
    sink = torch.zeros(blocks, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    out = {"metric": "dense MFMA peak, measured", "blocks": blocks,
           "waves_per_block": 4, "chains_per_wave": 8}
    for kind, name, fl_per, iters, spec in ((0, "bf16", 32768, 4000, 2500.0),
                                            (1, "fp8", 131072, 2000, 5000.0)):
        best, mhz = None, None
        for rep in range(6):
            a, b = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            a.record(stream)
            rc = lib.fa355_mfma_probe(kind, iters, blocks, clocks.data_ptr(),
                                      sink.data_ptr(), stream.cuda_stream)
            b.record(stream)
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"probe launch failed ({rc})")
            ms = a.elapsed_time(b)
            if rep == 0:
                continue            # first launch: code load and clock ramp
            c = clocks.cpu().tolist()
            clk = 100.0 * (c[1] - c[0]) / max(c[3] - c[2], 1)
            if best is None or ms < best:
                best, mhz = ms, clk
        flops = blocks * 4 * iters * 8 * fl_per
        tf = flops / (best * 1e-3) / 1e12
        out[name] = {"tflops": round(tf, 1), "spec_tflops": spec,
                     "frac_of_spec": round(tf / spec, 4), "ms": round(best, 3),
                     "shader_clock_mhz": round(mhz, 0)}
    print(json.dumps(out), flush=True)
    return 0


COEXEC_MODES = ["MFMA | MFMA", "MFMA | idle", "MFMA | FMA", "MFMA | EXP",
                "idle | FMA", "idle | EXP", "FMA | FMA", "LDS | LDS",
                "LDS-TR | LDS-TR", "MFMA+EXP | idle", "MFMA+FMA | idle",
                "MFMA | LDS", "MFMA | LDS-TR", "EXP | EXP", "LDS | idle",
                "MFMA+FMA | MFMA+FMA", "MFMA+EXP | MFMA+EXP", "BURST | BURST",
                "MIX2 | MIX2", "MIX4 | MIX4", "MIX6 | MIX6", "MIX8 | MIX8",
                "MIX5E1 | MIX5E1"]


def coexec_probe():
    """Co-issue of the execution units one CU shares: one workgroup of 8
    waves per CU (256 workgroups), waves w and w + 4 on the same SIMD, each
    running the role its mode gives it (libfa355_probe.so,
    fa355_coexec_probe); shader cycles per iteration, averaged over the
    workgroups, for waves 0-3 and 4-7, and the figures derived from them."""
    import ctypes
    import torch
    from io_aware_exact_04_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB)
    f = lib.fa355_coexec_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    blocks, iters = 256, 400
    cyc = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    sink = torch.zeros(blocks * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    per = {}
    for rep in range(2):
        for mode, name in enumerate(COEXEC_MODES):
            if f(mode, iters, blocks, cyc.data_ptr(), sink.data_ptr(),
                 stream.cuda_stream) != 0:
                raise RuntimeError("probe launch failed")
            torch.cuda.synchronize()
            c = cyc.view(blocks, 16).double().cpu()
            lo = c[:, 0:4].mean().item() / iters
            hi = c[:, 4:8].mean().item() / iters
            mhz = 100.0 * c[:, 0:8].sum().item() / max(c[:, 8:16].sum().item(), 1)
            if rep:                 # the first pass loads code and clocks up
                per[mode] = (lo, hi)
                print(json.dumps({"mode": mode, "roles": name,
                                  "cycles_per_iter_waves0_3": round(lo, 1),
                                  "cycles_per_iter_waves4_7": round(hi, 1),
                                  "shader_clock_mhz": round(mhz)}),
                      flush=True)
    mf = per[1][0] / 8
    derived = {
        "mfma_32x32x16_bf16_cycles": round(mf, 1),
        "fma_cycles_one_wave": round(per[4][1] / 64, 2),
        "fma_cycles_simd_two_waves": round(max(per[6]) / 128, 2),
        "exp_cycles_one_wave": round(per[5][1] / 16, 2),
        "exp_cycles_simd_two_waves": round(max(per[13]) / 32, 2),
        "lds_b128_bytes_per_cycle_cu": round(8 * 8 * 1024 / max(per[7]), 1),
        "lds_tr_b16_bytes_per_cycle_cu": round(8 * 8 * 512 / max(per[8]), 1),
        "mfma_slowdown_with_fma_partner": round(per[2][0] / per[1][0], 3),
        "fma_slowdown_with_mfma_partner": round(per[2][1] / per[4][1], 3),
        "mfma_slowdown_with_exp_partner": round(per[3][0] / per[1][0], 3),
        "exp_slowdown_with_mfma_partner": round(per[3][1] / per[5][1], 3),
        "mfma_slowdown_with_lds_partner": round(per[11][0] / per[1][0], 3),
        "mfma_slowdown_with_lds_tr_partner": round(per[12][0] / per[1][0], 3),
        "one_wave_mfma_plus_exp_vs_exp_alone":
            round(per[9][0] / (2 * per[5][1]), 3),
        "one_wave_mfma_plus_fma_vs_fma_alone":
            round(per[10][0] / (2 * per[4][1]), 3),
        # Both waves of a SIMD interleaving MFMAs with vector work: the
        # SIMD's MFMA pipe is busy 2 * 8 * mfma cycles per iteration.
        "two_waves_mfma_plus_fma_mfma_busy":
            round(2 * 8 * mf / max(per[15]), 3),
        "two_waves_mfma_plus_exp_mfma_busy":
            round(2 * 8 * mf / max(per[16]), 3),
        "two_waves_mfma_burst_then_fma_mfma_busy":
            round(2 * 8 * mf / max(per[17]), 3),
        # Both waves issuing k FMAs (and, for MIX5E1, one exponential)
        # after every MFMA.
        "two_waves_mix2_mfma_busy": round(2 * 8 * mf / max(per[18]), 3),
        "two_waves_mix4_mfma_busy": round(2 * 8 * mf / max(per[19]), 3),
        "two_waves_mix6_mfma_busy": round(2 * 8 * mf / max(per[20]), 3),
        "two_waves_mix8_mfma_busy": round(2 * 8 * mf / max(per[21]), 3),
        "two_waves_mix5e1_mfma_busy": round(2 * 8 * mf / max(per[22]), 3),
    }
    print(json.dumps({"metric": "co-issue probe, derived", **derived}),
          flush=True)
    return 0


def atomic_probe():
    """HBM cost of forming dQ inside the key-outer dK/dV kernel with fp32
    atomics: every 128-key workgroup adds one 64 x d fp32 partial tile per
    query tile its keys see (libfa355_probe.so, fa355_atomic_probe), at the
    headline shape B=2, H=32, N=4096, d=128 causal and at the dense
    B=4, H=16, N=1024, d=64 shape.  Median of 10 launches (HIP events on the
    launch stream) and the atomic bytes moved per second."""
    import ctypes
    import torch
    from io_aware_exact_04_amd import build as B
    lib = ctypes.CDLL(B.PROBE_LIB)
    f = lib.fa355_atomic_probe
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    for (BH, N, d, causal) in ((64, 4096, 128, True), (64, 1024, 64, False)):
        dq = torch.zeros(BH, N, d, dtype=torch.float32, device="cuda")
        nkb = (N + 127) // 128
        visits = sum(len(range(kb * 128 if causal else 0, N, 64))
                     for kb in range(nkb))
        nbytes = BH * visits * 64 * d * 4
        times = []
        for rep in range(12):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if f(BH, N, d, int(causal), dq.data_ptr(), stream.cuda_stream):
                raise RuntimeError("probe launch failed")
            e1.record(stream)
            torch.cuda.synchronize()
            if rep >= 2:
                times.append(e0.elapsed_time(e1) * 1e3)
        # Every element of a row block gets one 2^-10 per visiting key block.
        got = float(dq[0, -1, 0]) / 12 * 1024
        want = nkb
        us = float(np.median(times))
        print(json.dumps({"metric": "atomic probe", "BH": BH, "N": N, "d": d,
                          "causal": causal, "atomic_bytes": nbytes,
                          "median_us": round(us, 1),
                          "atomic_GB_per_s": round(nbytes / us / 1e3, 1),
                          "last_row_visits": got, "expected_visits": want}),
              flush=True)
    return 0


def bench_sweep(args):
    """Forward and backward over a grid of shapes ("Why is FlashAttention
    faster?", "Why FlashAttention is not always faster": speed-ups depend on
    sequence length, batch size, head dimension and causal mode): N from
    256 to 16384 at a fixed 16384 tokens per batch (B = 16384 / N, so short
    sequences come with large batches), H = 32, d in {64, 128}, dense and
    causal, bf16.  Inputs are seeded N(0,1) draws on the device (timing
    only; parity is the tests' business).  Each point: 3 untimed calls,
    then the median of 10 HIP-event timings of the forward and of the
    backward on the launch stream."""
    import torch
    import io_aware_exact_04_amd as fa
    H, tokens = 32, 16384
    stream = torch.cuda.current_stream()
    gen = torch.Generator(device="cuda").manual_seed(20240)
    rows = []
    for D in (64, 128):
        for causal in (False, True):
            for N in (256, 512, 1024, 2048, 4096, 8192, 16384):
                B = tokens // N
                q, k, v, do = (torch.randn(B, H, N, D, device="cuda",
                                           generator=gen).to(torch.bfloat16)
                               for _ in range(4))
                o = torch.empty_like(q)
                lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
                ws = torch.empty(max(fa.workspace_bytes(q), 16),
                                 dtype=torch.uint8, device="cuda")
                grads = tuple(torch.empty_like(q) for _ in range(3))
                scale = 1.0 / np.sqrt(D)

                def fwd():
                    fa.fa_fwd(q, k, v, scale, causal, out=o, lse=lse)

                def bwd():
                    fa.fa_bwd(q, k, v, o, lse, do, scale, causal,
                              workspace=ws, out=grads)

                def timed(fn):
                    for _ in range(3):
                        fn()
                    evs = [(torch.cuda.Event(enable_timing=True),
                            torch.cuda.Event(enable_timing=True))
                           for _ in range(10)]
                    for a, b in evs:
                        a.record(stream)
                        fn()
                        b.record(stream)
                    torch.cuda.synchronize()
                    return float(np.median([a.elapsed_time(b)
                                            for a, b in evs]))
                f_ms = timed(fwd)
                b_ms = timed(bwd)
                ff = cost.fwd_flops(B, H, N, D, causal)
                bf = cost.bwd_flops(B, H, N, D, causal)
                row = {"sweep": "fwd+bwd", "B": B, "H": H, "N": N, "d": D,
                       "causal": causal, "fwd_ms": round(f_ms, 4),
                       "bwd_ms": round(b_ms, 4),
                       "fwd_tflops": round(ff / f_ms / 1e9, 1),
                       "bwd_tflops": round(bf / b_ms / 1e9, 1),
                       "fwd_bwd_tflops": round((ff + bf) / (f_ms + b_ms)
                                               / 1e9, 1),
                       "fwd_bwd_frac_peak": round((ff + bf) / (f_ms + b_ms)
                                                  / 1e9 / PEAK_BF16_TFLOPS,
                                                  4)}
                rows.append(row)
                print(json.dumps(row), flush=True)
                del q, k, v, do, o, lse, ws, grads
    return 0


def bench_fp8(args):
    """FP8 forward with incoherent processing on the headline shape (B=2,
    H=32, N=4096, d=128, causal, bf16 in and out): the quantisation kernel
    (Hadamard rotation of Q and K, per-64-row E4M3 quantisation of Q, K, V;
    HBM-bound) and the FP8 attention kernel (FP8 matrix cores), timed apart
    with HIP events on the launch stream, and the bf16 forward on the same
    inputs for comparison.  Counted FLOPs as for the bf16 forward."""
    import torch
    import io_aware_exact_04_amd as fa
    w = W.get("c3")
    inp = W.make_inputs(w)
    q, k, v = (W.to_torch(inp[x], "bf16", "cuda") for x in ("q", "k", "v"))
    signs = W.hadamard_signs(w.D, 33)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fp8_layout(q).bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    Ev = torch.cuda.Event

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fp8_quantize(q, k, v, signs, True, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_fwd_fp8_quantized(ws, o, lse, w.scale, True, True)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[Ev(enable_timing=True) for _ in range(3)]
              for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    quant_us = float(np.mean([e[0].elapsed_time(e[1]) for e in events])) * 1e3
    attn_us = float(np.mean([e[1].elapsed_time(e[2]) for e in events])) * 1e3
    # bf16 forward on the same inputs, same stream.
    o2 = torch.empty_like(q)
    for _ in range(args.warmup):
        fa.fa_fwd(q, k, v, w.scale, True, out=o2, lse=lse)
    ev2 = [(Ev(enable_timing=True), Ev(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in ev2:
        a.record(stream)
        fa.fa_fwd(q, k, v, w.scale, True, out=o2, lse=lse)
        b.record(stream)
    torch.cuda.synchronize()
    bf16_us = float(np.mean([a.elapsed_time(b) for a, b in ev2])) * 1e3

    fl = cost.fwd_flops(w.B, w.H, w.N, w.D, True, None, 128)
    ms_per_step = wall / args.steps * 1e3
    attn_tf = fl / (attn_us * 1e-6) / 1e12
    # Quantisation bytes: bf16 Q, K, V read; E4M3 codes and scales written.
    lay = fa.fp8_layout(q)
    qbytes = 3 * q.numel() * 2 + lay.bytes
    line = {
        "metric": "FP8 attention forward TFLOP/s (quantise + FP8 kernel), "
                  "N=4096 d=128 causal",
        "value": round(fl / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) inputs, see workloads)",
        "config": {"workload": "fp8: " + describe(w) + ", Hadamard-rotated "
                   "Q, K; E4M3 per 64-row block; E4M3 P",
                   "counted_gflop_fwd": round(fl / 1e9, 3)},
        "kernels_avg_us": {"fp8_quantize": round(quant_us, 2),
                           "fwd_fp8": round(attn_us, 2),
                           "fwd_bf16_same_inputs": round(bf16_us, 2)},
        "fwd_fp8_tflops": round(attn_tf, 2),
        "speedup_over_bf16_forward": round(bf16_us / (quant_us + attn_us), 3),
        "quantize_gbs": round(qbytes / (quant_us * 1e-6) / 1e9, 1),
        "roofline": {"bound": "mfma", "kernel": "fwd_fp8",
                     "achieved": round(attn_tf, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": None, "avg_launch_us": round(attn_us, 2),
                     "algorithmic_flops_per_launch": fl},
    }
    print(json.dumps(line), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not "
              "supported (heads are independent; see the sharding notes)",
              file=sys.stderr)
        return 2
    import torch
    if args.mfma_probe:
        return mfma_probe()
    if args.coexec_probe:
        return coexec_probe()
    if args.atomic_probe:
        return atomic_probe()
    if args.sweep:
        return bench_sweep(args)
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 3}), flush=True)
        return 0
    if args.workload in W.KV_WORKLOADS:
        return bench_decode(args)
    if args.workload == "varlen":
        return bench_varlen(args)
    if args.workload == "fp8":
        return bench_fp8(args)
    if args.workload == "drop":
        return bench_dropout(args)
    if args.workload == "pad":
        return bench_padding(args)
    import io_aware_exact_04_amd as fa

    w = W.get(args.workload)
    inp = W.make_inputs(w)
    dev = "cuda"
    q, k, v, do = (W.to_torch(inp[x], w.dtype, dev) for x in
                   ("q", "k", "v", "do"))
    mask = (torch.from_numpy(inp["block_mask"]).to(dev)
            if inp["block_mask"] is not None else None)
    mb = w.mask_block or 128
    ws = torch.empty(max(fa.workspace_bytes(q), 16), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    Ev = torch.cuda.Event

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, w.scale, w.causal, mask, mb, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        if not w.backward:
            return

        def between(i):
            if ev is not None:
                ev[2 + i].record(stream)
        fa.fa_bwd(q, k, v, o, lse, do, w.scale, w.causal, mask, mb,
                  workspace=ws, stages=(0, 1), between=between)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    clock_before = shader_clock_mhz()
    events = [[Ev(enable_timing=True) for _ in range(4)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    clock_after = shader_clock_mhz()

    def times(a, b):
        return [e[a].elapsed_time(e[b]) for e in events]

    def avg(a, b):
        return float(np.mean(times(a, b)))

    fwd_ms = avg(0, 1)
    fwd_fl = cost.fwd_flops(w.B, w.H, w.N, w.D, w.causal, inp["block_mask"],
                            mb)
    out = {"fwd_ms": fwd_ms, "fwd_tflops": fwd_fl / fwd_ms / 1e9}
    kernels = {"fwd": fwd_ms * 1e3}
    # Spread over the timed steps (HIP events on the launch stream), per
    # kernel in microseconds and for the whole step in milliseconds.
    spans = {"fwd": (0, 1)}
    if w.backward:
        spans.update(bwd_dq=(1, 2), bwd_dkdv=(2, 3))
    kernel_spread = {k_: {s_: round(v_ * 1e3, 2) for s_, v_ in
                          spread(times(*ab)).items()}
                     for k_, ab in spans.items()}
    step_spread = spread(times(0, 3 if w.backward else 1))
    total_fl = fwd_fl
    if w.backward:
        bwd_fl = cost.bwd_flops(w.B, w.H, w.N, w.D, w.causal,
                                inp["block_mask"], mb)
        dq_ms, dkdv_ms = avg(1, 2), avg(2, 3)
        bwd_ms = avg(1, 3)
        kernels.update(bwd_dq=dq_ms * 1e3, bwd_dkdv=dkdv_ms * 1e3)
        total_fl += bwd_fl
        out.update(bwd_ms=bwd_ms, bwd_tflops=bwd_fl / bwd_ms / 1e9,
                   fwd_bwd_ms=fwd_ms + bwd_ms,
                   fwd_bwd_tflops=total_fl / (fwd_ms + bwd_ms) / 1e9)
    ms_per_step = wall / args.steps * 1e3
    value = total_fl / (ms_per_step / 1e3) / 1e12

    # Dominant kernel: the one with the largest average launch time.
    dom = max(kernels, key=kernels.get)
    dom_us = kernels[dom]
    bwd_fl = (cost.bwd_flops(w.B, w.H, w.N, w.D, w.causal,
                             inp["block_mask"], mb) if w.backward else 0.0)
    executed_fl = None
    if dom == "fwd":
        dom_fl = fwd_fl
    elif dom == "bwd_dkdv":
        dom_fl = bwd_fl * 4 / 5
    elif dom == "bwd_dq":
        dom_fl = bwd_fl / 5
        executed_fl = bwd_fl * 3 / 5
    else:
        dom_fl = None
    traffic = None
    try:
        with open(args.traffic_json) as f:
            tj = json.load(f).get(w.name, {})
        # Counters describe one build of the kernels: ignore them once the
        # sources have changed.
        if tj.get("source_sha256_16") == source_digest():
            rec = tj.get(dom)
            if rec:
                traffic = rec.get("bytes_per_dispatch")
    except (OSError, ValueError):
        pass
    if w.dtype == "bf16" and dom_fl is not None:
        achieved = dom_fl / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": dom,
                    "achieved": round(achieved, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic,
                    "avg_launch_us": round(dom_us, 2),
                    "algorithmic_flops_per_launch": dom_fl}
        if executed_fl is not None:
            roofline["executed_flops_per_launch"] = executed_fl
    else:
        achieved = (dom_fl or 0) / (dom_us * 1e-6) / 1e12
        roofline = {"bound": "alu", "kernel": dom,
                    "achieved": round(achieved, 3),
                    "peak": PEAK_FP32_VALU_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_FP32_VALU_TFLOPS, 4),
                    "traffic": traffic, "avg_launch_us": round(dom_us, 2)}

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, see workloads)",
        "config": {"workload": describe(w), "B": w.B, "H": w.H, "N": w.N,
                   "d": w.D, "causal": w.causal,
                   "block_mask": w.has_mask,
                   "counted_gflop_fwd": round(fwd_fl / 1e9, 3),
                   "counted_gflop_fwd_bwd": round(total_fl / 1e9, 3)},
        "fwd_tflops": round(out["fwd_tflops"], 2),
        "fwd_frac_peak": round(out["fwd_tflops"] / PEAK_BF16_TFLOPS, 4),
        "fwd_ms": round(fwd_ms, 4),
        "kernels_avg_us": {k_: round(v_, 2) for k_, v_ in kernels.items()},
        "kernels_spread_us": kernel_spread,
        "step_ms_spread": step_spread,
        "shader_clock_mhz": {"before": clock_before, "after": clock_after},
        "roofline": roofline,
    }
    if w.backward:
        line.update(bwd_tflops=round(out["bwd_tflops"], 2),
                    fwd_bwd_tflops=round(out["fwd_bwd_tflops"], 2),
                    fwd_bwd_frac_peak=round(out["fwd_bwd_tflops"] /
                                            PEAK_BF16_TFLOPS, 4),
                    bwd_ms=round(out["bwd_ms"], 4))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
