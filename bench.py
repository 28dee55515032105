#!/usr/bin/env python3
"""Throughput of the block-scaled FP4 quantization path on one MI355X.

Headline workload (one "step" = one pass of the hot path over one batch):
MXFP4 quantization of MoE expert activations, 16384 tokens x 4096 hidden,
bf16 Student-t(4) values, 32-element blocks with E8M0 scales:
  1. rollout side: RTN quantize of the rollout copy x_r,
  2. guide_pack of its codes and scales (1 mantissa bit + block scale),
  3. trainer side: guided quantize of x with that guide,
  4. dequantize of the guided codes to bf16,
  5. stochastic rounding (Philox, key 1) of an activation batch of the same
     shape (the previous batch's x, so no input is re-read from the last-level
     cache within a step).
The five kernels run in that order on one stream.  Kernels 1-4 form a
dependent chain and kernel 5 depends on none of them; ``--streams 2`` runs it
on a second stream (default priority) beside the chain.  Both orders are timed
on every run and reported; ``value`` uses the one ``--streams`` selects.
``value`` = algorithmic bytes of the step / step time, in GB/s, measured with
HIP events around K whole steps.  Every timed region is preceded by 100 ms of
untimed launches of the same work (the shader clock idles low while the host
generates data, and takes tens of milliseconds of load to climb), then the W
warm-up steps.  Inputs are resident in HBM before timing; a
rotating pool of input sets (768 MiB) keeps the 256 MB Infinity Cache from
serving re-reads across steps.

Per kernel, two durations are reported: with events around every launch inside
the steps, and as back-to-back launches of that kernel alone (events around
the loop).  The roofline entry is for the kernel with the largest share of the
step, by its back-to-back duration, which compares directly with rocprofv3's
kernel durations; a second entry covers the largest workload's quantize kernel
(uniform grid + RHT16 + SR, 65536x8192).  Means come with the 10th, 50th and 90th
percentiles of single launches (and of single steps).  The other workloads (NVFP4 activation 4096x2048,
KV cache at 131072 tokens, one deep guidance-cache layer, uniform grid + RHT16
+ SR on a 65536x8192 GEMM operand) are timed back to back and reported under
"workloads", and so is the MXFP4 matrix product of one deep layer's
activations [8192, 4096] with one expert weight [1536 out, 4096 in], both
quantized by the library, reported as TFLOP/s against the dense FP4 matrix
peak.  The CPU baseline is the oracle timed on a bounded row sample of the
headline step, on one host thread and on all host threads of one GPU's share
(at most 16, rows split between them).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick] [--streams 1|2]
                       [--workload all|c1|c3|c4|c5|gemm]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, GB/s
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak (no sparsity), TFLOP/s
SETTLE_MS = 100.0  # untimed load before every timed region (shader clock ramp)


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2))
    ap.add_argument("--quick", action="store_true", help="headline workload only, no CPU baseline")
    ap.add_argument("--gemm-only", action="store_true", help="same as --workload gemm")
    ap.add_argument("--workload", default="all", choices=("all", "c1", "c3", "c4", "c5", "gemm"),
                    help="all: the headline step, then every other workload; otherwise only that workload "
                         "(one JSON line of its figures, for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of the CPU-baseline sample")
    ap.add_argument("--config-iters", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed load before every timed region (shorter under a profiler: fewer dispatches)")
    return ap.parse_args()


# ---------------------------------------------------------------- helpers
def to_dev(u16: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


class KernelTimer:
    """Per-kernel HIP-event timing on the current stream (events recorded between launches)."""

    def __init__(self):
        self.events = []  # (name, start, end)

    def run(self, name, fn):
        import torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        out = fn()
        e.record()
        self.events.append((name, s, e))
        return out

    def summary(self):
        """name -> (mean ms, launches, (p10, median, p90) ms)."""
        per = {}
        for name, s, e in self.events:
            per.setdefault(name, []).append(s.elapsed_time(e))
        return {k: (sum(v) / len(v), len(v), tuple(float(q) for q in np.percentile(v, [10, 50, 90])))
                for k, v in per.items()}


def settle(torch, fn, ms=None):
    """Untimed calls of fn(i) until the GPU has run them for `ms` milliseconds: the shader clock
    idles low between workloads (host-side data generation) and needs tens of milliseconds of load
    to climb, so shorter warm-ups time a partly down-clocked GPU."""
    ms = SETTLE_MS if ms is None else ms
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(4):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return


_last_spread = None   # (p10, median, p90) ms of the latest back_to_back, picked up by report()


def back_to_back(torch, fn, reps, warm=2):
    """Average ms of `fn(i)` over `reps` consecutive launches on the current stream, after a settle.
    A second pass times up to 50 launches one by one between events, for the spread."""
    global _last_spread
    settle(torch, fn)
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(min(reps, 50))]
    for i, (x, y) in enumerate(ev):
        x.record()
        fn(i)
        y.record()
    torch.cuda.synchronize()
    _last_spread = tuple(float(q) for q in np.percentile([x.elapsed_time(y) for x, y in ev], [10, 50, 90]))
    return ms


def graph_time(torch, fn, reps, check):
    """Average ms per launch of `reps` launches of fn(i) captured in one HIP graph and replayed, so
    that host-side launch cost (several microseconds per call from Python) does not hide the
    duration of small kernels.  check() compares the outputs with an eager run; it follows every
    replay (two untimed, one timed).  Returns (ms, all checks passed)."""
    settle(torch, fn)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    ok = True
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        ok = ok and bool(check())
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    ok = ok and bool(check())
    del g
    return a.elapsed_time(b) / reps, ok


def source_sha():
    h = hashlib.sha256()
    for f in ["device.h", "internal.h", "quantize.hip", "misc.hip", "abi.hip"]:
        with open(os.path.join(HERE, "precision_rl_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_key: str, sha: str):
    """HBM traffic per launch measured with rocprofv3 --pmc (FETCH_SIZE / WRITE_SIZE),
    scaled by the copy-kernel calibration; valid only for the same kernel sources."""
    path = os.path.join(HERE, "profiles", "hbm_traffic.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == kernel_key and cells[1] == sha:
            try:
                return float(cells[3])
            except ValueError:
                return None
    return None


def take_spread():
    """The (p10, median, p90) of the latest back_to_back call, in microseconds, and forget it."""
    global _last_spread
    sp, _last_spread = _last_spread, None
    return None if sp is None else [round(q * 1e3, 2) for q in sp]


def report(ms, nbytes, n, ceiling=None):
    """Rates for a mean launch time ms; with the spread of the back_to_back call that produced it
    (per-launch events, which add a little time of their own)."""
    gbs = nbytes / (ms * 1e-3) / 1e9
    r = {"us": round(ms * 1e3, 2), "bytes": int(nbytes), "GBps": round(gbs, 1),
         "Gelem_per_s": round(n / (ms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    if ceiling:
        r["frac_copy_ceiling"] = round(gbs / ceiling, 4)
    sp = take_spread()
    if sp is not None:
        r["us_p10_median_p90_single_launch"] = sp
    return r


# ---------------------------------------------------------------- copy ceiling
def copy_ceiling(torch, fq, mib=256, reps=20):
    """The library's plain streaming copy (16 B per lane): the practical bandwidth reference."""
    n = mib * (1 << 20)
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1)
    ms = back_to_back(torch, lambda i: fq.fp4_stream_copy(bufs[(2 * i) % 4], bufs[(2 * i + 1) % 4]), reps)
    return {"bytes_per_launch": 2 * n, "us": round(ms * 1e3, 2), "GBps": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "us_p10_median_p90_single_launch": take_spread()}


# ---------------------------------------------------------------- headline step
def headline(args, fq, torch, W, ceiling):
    rows, cols = W.c2_shape()
    n = rows * cols
    log(f"generating C2 {rows}x{cols} Student-t(4) ...")
    x_h, xr_h = W.c2_pair(rows, cols, seed=1)
    cfg_rtn = fq.Fp4Config(format=fq.MXFP4)
    # SR quantizes the gradient for a later product: no kernel of the step reads its output, which
    # therefore streams past the caches (stream_out); the others' outputs are read by the next kernel
    cfg_sr = fq.Fp4Config(format=fq.MXFP4, rounding=fq.SR, sr_seed=W.C2_SR_SEED, stream_out=True)
    P = 3  # rotating input sets: 3 x 256 MiB
    x0, xr0 = to_dev(x_h), to_dev(xr_h)
    xs = [x0] + [torch.roll(x0, shifts=(s * 977), dims=0) for s in range(1, P)]
    xrs = [xr0] + [torch.roll(xr0, shifts=(s * 977), dims=0) for s in range(1, P)]
    B = 32
    u8 = lambda k: torch.empty(k, dtype=torch.uint8, device="cuda")
    outs = [dict(rc=u8(n // 2), rs=u8(n // B), gb=u8(n // 8), gs=u8(n // B), gc=u8(n // 2), gsc=u8(n // B),
                 sc=u8(n // 2), ss=u8(n // B), dq=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"))
            for _ in range(P)]
    chain = ["quantize_rtn", "guide_pack", "quantize_guided", "dequantize_bf16"]

    def step_fns(k):
        s = k % P
        o = outs[s]
        return {
            "quantize_rtn": lambda: fq.fp4_quantize(xrs[s], cfg_rtn, None, codes=o["rc"], scales=o["rs"]),
            "guide_pack": lambda: fq.guide_pack(o["rc"], o["rs"], cfg_rtn, rows, cols, bits=o["gb"], gscales=o["gs"]),
            "quantize_guided": lambda: fq.fp4_quantize_guided(xs[s], cfg_rtn, o["gb"], o["gs"], None,
                                                              codes=o["gc"], scales=o["gsc"]),
            "dequantize_bf16": lambda: fq.fp4_dequantize(o["gc"], o["gsc"], cfg_rtn, rows, cols, None, out=o["dq"]),
            "quantize_sr": lambda: fq.fp4_quantize(xs[(s + 2) % P], cfg_sr, None, codes=o["sc"], scales=o["ss"]),
        }

    bytes_per = {  # algorithmic bytes per element of each kernel (MXFP4, B = 32)
        "quantize_rtn": 2 + 0.5 + 1 / 32,
        "guide_pack": 0.5 + 1 / 32 + 1 / 8 + 1 / 32,
        "quantize_guided": 2 + 1 / 8 + 1 / 32 + 0.5 + 1 / 32,
        "dequantize_bf16": 0.5 + 1 / 32 + 2,
        "quantize_sr": 2 + 0.5 + 1 / 32,
    }
    step_bytes = sum(bytes_per.values()) * n
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()  # default priority

    def step(k, streams):
        f = step_fns(k)
        if streams == 2:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                f["quantize_sr"]()
            for name in chain:
                f[name]()
            main.wait_stream(side)
        else:
            for name in chain + ["quantize_sr"]:
                f[name]()

    def timed_steps(streams):
        settle(torch, lambda k: step(k, streams))
        for k in range(args.warmup):
            step(k, streams)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for k in range(args.steps):
            step(k, streams)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    log("timing steps ...")
    ms_serial = timed_steps(1)
    ms_two = timed_steps(2)
    ms_step = ms_two if args.streams == 2 else ms_serial
    # each step on its own between events (a separate pass): the spread of step times
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record()
        step(k, args.streams)
        ev[k][1].record()
    torch.cuda.synchronize()
    step_pct = [round(float(q) * 1e3, 2) for q in np.percentile([a.elapsed_time(b) for a, b in ev], [10, 50, 90])]
    # events around every kernel inside serialized steps
    timer = KernelTimer()
    for k in range(args.steps):
        for name, fn in step_fns(k).items():
            timer.run(name, fn)
    torch.cuda.synchronize()
    kernels = {}
    # in-step figures are medians: a launch timed between two events also times any host stall
    # between the first event and the launch (one 34 ms stall once made a 10 us kernel's mean 352 us)
    for name, (ms, cnt, pct) in timer.summary().items():
        kernels[name] = dict(report(pct[1], bytes_per[name] * n, n, ceiling), launches=cnt,
                             us_mean=round(ms * 1e3, 2), us_p10_median_p90=[round(q * 1e3, 2) for q in pct])
    # back-to-back launches of each kernel alone: the roofline figure.  Inputs and outputs rotate over Q
    # sets (the codes and guides the step produced, copied), so that no set comes round again within more
    # than 1 GiB of traffic: neither reads nor writes can be served by the 256 MB Infinity Cache.
    # (Reusing one output buffer lets that cache absorb the writes: 16384 x 4096 MXFP4 RTN measured
    # 27.2 us with its outputs rotated over three sets, 102 MB, and 30.2 us over twelve.)
    Q = 12
    bq = [dict(rc=outs[j % P]["rc"].clone(), rs=outs[j % P]["rs"].clone(), gb=outs[j % P]["gb"].clone(),
               gs=outs[j % P]["gs"].clone(), gc=outs[j % P]["gc"].clone(), gsc=outs[j % P]["gsc"].clone(),
               sc=u8(n // 2), ss=u8(n // B)) for j in range(Q)]
    dqq = [torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
    alone = {
        "quantize_rtn": lambda i: fq.fp4_quantize(xrs[i % P], cfg_rtn, None, codes=bq[i % Q]["rc"],
                                                  scales=bq[i % Q]["rs"]),
        "guide_pack": lambda i: fq.guide_pack(bq[i % Q]["rc"], bq[i % Q]["rs"], cfg_rtn, rows, cols,
                                              bits=bq[i % Q]["gb"], gscales=bq[i % Q]["gs"]),
        "quantize_guided": lambda i: fq.fp4_quantize_guided(xs[i % P], cfg_rtn, bq[i % Q]["gb"], bq[i % Q]["gs"], None,
                                                            codes=bq[i % Q]["gc"], scales=bq[i % Q]["gsc"]),
        "dequantize_bf16": lambda i: fq.fp4_dequantize(bq[i % Q]["gc"], bq[i % Q]["gsc"], cfg_rtn, rows, cols, None,
                                                       out=dqq[i % 4]),
        "quantize_sr": lambda i: fq.fp4_quantize(xs[(i + 2) % P], cfg_sr, None, codes=bq[i % Q]["sc"],
                                                 scales=bq[i % Q]["ss"]),
    }
    for name in kernels:
        ms = back_to_back(torch, alone[name], args.steps)
        r = report(ms, bytes_per[name] * n, n, ceiling)
        kernels[name]["us_back_to_back"] = r["us"]
        kernels[name]["GBps_back_to_back"] = r["GBps"]
        kernels[name]["frac_hbm_peak_back_to_back"] = r["frac_hbm_peak"]
        kernels[name]["us_p10_median_p90_single_launch"] = r.get("us_p10_median_p90_single_launch")
    # guided fake quantization (quantize -> bf16 in one pass), the QAT forward op
    ms = back_to_back(torch, lambda i: fq.fp4_fake_quantize(xs[i % P], cfg_rtn, None, bq[i % Q]["gb"],
                                                            bq[i % Q]["gs"], out=dqq[i % 4]), args.steps)
    fake = report(ms, (2 + 1 / 8 + 1 / 32 + 2) * n, n, ceiling)
    # full-code guided diagnostic: x against the rollout's RTN codes of x_r
    cnt = torch.empty(3, dtype=torch.int64, device="cuda")
    for j in range(Q):   # the rollout codes of x_r again (the sets were overwritten by the timing above)
        fq.fp4_quantize(xrs[j % P], cfg_rtn, None, codes=bq[j]["rc"], scales=bq[j]["rs"])
    ms = back_to_back(torch, lambda i: fq.fp4_guide_mismatch(xs[i % P], cfg_rtn, bq[i % Q]["rc"], bq[i % Q]["rs"],
                                                             None, out=cnt), args.steps)
    diag = dict(report(ms, (2 + 0.5 + 1 / 32) * n, n, ceiling),
                **mismatch_counts(fq, xs[0], cfg_rtn, bq[0]["rc"], bq[0]["rs"], None))
    del bq, dqq
    return dict(rows=rows, cols=cols, n=n, ms_step=ms_step, ms_serial=ms_serial, ms_two=ms_two, step_bytes=step_bytes,
                step_us_p10_median_p90=step_pct,
                kernels=kernels, bytes_per=bytes_per, x_h=x_h, xr_h=xr_h, outs=outs[0], fake=fake, diag=diag)


def parity_sample(torch, h, oracle_mod, rows_s=64):
    """Compare the headline step's slot-0 outputs with the oracle on the first rows."""
    O = oracle_mod
    cols = h["cols"]
    o = h["outs"]
    n_s = rows_s * cols
    oc = O.Cfg(format=O.MXFP4)
    rc, rs = O.quantize(oc, O.RTN, h["xr_h"][:rows_s])
    gb, gs = O.guide_pack(oc, rc, rs, rows_s, cols)
    gc, gsc = O.quantize(oc, O.GUIDED, h["x_h"][:rows_s], guide_bits=gb, guide_scales=gs)
    dq = O.dequantize(oc, gc, gsc, 1.0, rows_s, cols, out_bf16=True)
    ok = (o["rc"][: n_s // 2].cpu().numpy() == rc).all() and (o["gb"][: n_s // 8].cpu().numpy() == gb).all()
    ok = ok and (o["gc"][: n_s // 2].cpu().numpy() == gc).all() and (o["gsc"][: n_s // 32].cpu().numpy() == gsc).all()
    ok = ok and (o["dq"][:rows_s].contiguous().view(torch.int16).cpu().numpy().reshape(-1) == dq.view(np.int16)).all()
    return bool(ok)


def _oracle_step_rows(O, W, h, r0, r1):
    """The five kernels of the step, by the oracle, on rows [r0, r1) (the SR counter follows the rows)."""
    cols = h["cols"]
    x, xr = h["x_h"][r0:r1], h["xr_h"][r0:r1]
    oc = O.Cfg(format=O.MXFP4)
    osr = O.Cfg(format=O.MXFP4, sr_seed=W.C2_SR_SEED, sr_offset=r0 * cols // 16)
    R = r1 - r0
    rc, rs = O.quantize(oc, O.RTN, xr)
    gb, gs = O.guide_pack(oc, rc, rs, R, cols)
    gc, gsc = O.quantize(oc, O.GUIDED, x, guide_bits=gb, guide_scales=gs)
    O.dequantize(oc, gc, gsc, 1.0, R, cols, out_bf16=True)
    O.quantize(osr, O.SR, x)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, W, oracle_mod, h, threads=1, runs=3):
    """The oracle (unchanged) on rows [0, R) of the headline step, on `threads` host threads with the
    rows split evenly between them (the oracle's C calls release the interpreter lock); the median
    of `runs` timed runs after one untimed run."""
    import concurrent.futures as cf
    R = min(args.cpu_rows, h["rows"])
    cols = h["cols"]
    cuts = [R * k // threads for k in range(threads + 1)]

    def one():
        t = time.perf_counter()
        if threads == 1:
            _oracle_step_rows(oracle_mod, W, h, 0, R)
        else:
            with cf.ThreadPoolExecutor(threads) as ex:
                list(ex.map(lambda k: _oracle_step_rows(oracle_mod, W, h, cuts[k], cuts[k + 1]), range(threads)))
        return time.perf_counter() - t
    one()
    times = sorted(one() for _ in range(runs))
    dt = times[len(times) // 2]
    b = sum(h["bytes_per"].values()) * R * cols
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"rows 0..{R} of the 16384x4096 workload ({R * cols} elements), all five kernels "
                      f"of the step, {threads} thread(s) over row ranges; median of {runs} runs after one "
                      f"untimed run: {dt:.2f} s (runs {', '.join(f'{x:.2f}' for x in times)} s); host: "
                      f"{os.cpu_count()} logical CPUs, {_cpu_model()}"}


# ---------------------------------------------------------------- other workloads
def mismatch_counts(fq, x, cfg, rcodes, rscales, ts):
    """Full-code guided diagnostic of x against a rollout's codes: how often the 1-bit guide
    cannot reproduce the rollout's codeword (non-adjacent) or its code (mismatched), and how often
    the trainer's own RTN quantization of x (its own tensor scale for NVFP4) differs from the
    rollout's code: the training/rollout mismatch that guided rounding removes."""
    n, nonadj, mism = (int(v) for v in fq.fp4_guide_mismatch(x, cfg, rcodes, rscales, ts).cpu())
    own_ts = fq.fp4_tensor_scale(x, cfg) if cfg.format == fq.NVFP4 else None
    own, _ = fq.fp4_quantize(x, cfg, own_ts)
    d = own ^ rcodes
    rtn = int(((d & 0xF) != 0).sum().item() + ((d >> 4) != 0).sum().item())
    return {"elements": n, "non_adjacent": nonadj, "mismatched": mism,
            "non_adjacent_frac": nonadj / max(n, 1), "mismatched_frac": mism / max(n, 1),
            "rtn_differs": rtn, "rtn_differs_frac": rtn / max(n, 1)}


def _u8(torch):
    return lambda k: torch.empty(k, dtype=torch.uint8, device="cuda")


def wl_c1(args, fq, torch, W, ceiling):
    """NVFP4 activation 4096x2048 (16 MiB): inputs rotate over 32 copies (512 MiB) and outputs over 64 sets
    (368 MB), so that the Infinity Cache serves neither."""
    it = args.config_iters
    u8 = _u8(torch)
    rows, cols = W.c1_shape()
    n = rows * cols
    log("NVFP4 activation 4096x2048 ...")
    x0, xr0 = to_dev(W.c1_x(rows, cols)), to_dev(W.c1_rollout(rows, cols))
    cfg = fq.Fp4Config()
    P, R = 32, 64
    xs = [torch.roll(x0, s * 61, 0) for s in range(P)]
    xrs = [torch.roll(xr0, s * 61, 0) for s in range(P)]
    tss = [fq.fp4_tensor_scale(xr, cfg) for xr in xrs]
    guides = [fq.fp4_quantize(xrs[s], cfg, tss[s], emit=True) for s in range(P)]
    oc, os_, ob = [u8(n // 2) for _ in range(R)], [u8(n // 16) for _ in range(R)], [u8(n // 8) for _ in range(R)]
    tso = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in range(R)]
    r = {}
    r["tensor_scale"] = report(back_to_back(torch, lambda i: fq.fp4_tensor_scale(xs[i % P], cfg, out=tso[i % R]), it), 2 * n, n, ceiling)
    r["quantize_rtn"] = report(back_to_back(torch, lambda i: fq.fp4_quantize(xs[i % P], cfg, tss[i % P], codes=oc[i % R], scales=os_[i % R]), it), 2.5625 * n, n, ceiling)
    r["quantize_rtn_emit"] = report(back_to_back(torch, lambda i: fq.fp4_quantize(xs[i % P], cfg, tss[i % P], emit=True, codes=oc[i % R], scales=os_[i % R], bits=ob[i % R]), it), 2.6875 * n, n, ceiling)
    r["quantize_guided"] = report(back_to_back(torch, lambda i: fq.fp4_quantize_guided(xs[i % P], cfg, guides[i % P][2], guides[i % P][1], tss[i % P], codes=oc[i % R], scales=os_[i % R]), it), 2.75 * n, n, ceiling)
    cnt = torch.empty(3, dtype=torch.int64, device="cuda")
    r["guide_mismatch"] = report(back_to_back(torch, lambda i: fq.fp4_guide_mismatch(xs[i % P], cfg, guides[i % P][0], guides[i % P][1], tss[i % P], out=cnt), it), 2.5625 * n, n, ceiling)
    r["guide_mismatch_counts"] = mismatch_counts(fq, xs[0], cfg, guides[0][0], guides[0][1], tss[0])
    # the same kernels as one graph of launches: at 16 MiB a call from Python costs about as much
    # host time as the kernel runs, so the eager figures above are bound by the host
    gr = max(it, 64)
    last = gr - 1

    def same(*pairs):
        return all(torch.equal(a, b) for a, b in pairs)
    L, Lo = last % P, last % R
    ms, ok = graph_time(torch, lambda i: fq.fp4_tensor_scale(xs[i % P], cfg, out=tso[i % R]), gr,
                        lambda: same((tso[Lo], fq.fp4_tensor_scale(xs[L], cfg))))
    r["tensor_scale_graph"] = dict(report(ms, 2 * n, n, ceiling), replays_match_eager=ok)
    ms, ok = graph_time(torch, lambda i: fq.fp4_quantize(xs[i % P], cfg, tss[i % P], codes=oc[i % R], scales=os_[i % R]), gr,
                        lambda: same(*zip((oc[Lo], os_[Lo]), fq.fp4_quantize(xs[L], cfg, tss[L]))))
    r["quantize_rtn_graph"] = dict(report(ms, 2.5625 * n, n, ceiling), replays_match_eager=ok)
    ms, ok = graph_time(torch, lambda i: fq.fp4_quantize(xs[i % P], cfg, tss[i % P], emit=True, codes=oc[i % R],
                                                         scales=os_[i % R], bits=ob[i % R]), gr,
                        lambda: same(*zip((oc[Lo], os_[Lo], ob[Lo]), fq.fp4_quantize(xs[L], cfg, tss[L], emit=True))))
    r["quantize_rtn_emit_graph"] = dict(report(ms, 2.6875 * n, n, ceiling), replays_match_eager=ok)
    ms, ok = graph_time(torch, lambda i: fq.fp4_quantize_guided(xs[i % P], cfg, guides[i % P][2], guides[i % P][1],
                                                                tss[i % P], codes=oc[i % R], scales=os_[i % R]), gr,
                        lambda: same(*zip((oc[Lo], os_[Lo]), fq.fp4_quantize_guided(xs[L], cfg, guides[L][2],
                                                                                     guides[L][1], tss[L]))))
    r["quantize_guided_graph"] = dict(report(ms, 2.75 * n, n, ceiling), replays_match_eager=ok)
    # the tensor scale in one launch (workspace), alone and followed by the RTN quantize that uses it.
    # End to end the task's algorithmic bytes are those of one pass: x read once and the codes and
    # scales written (2.5625 bytes per element); the two- and four-launch forms read x twice
    ws = fq.tensor_scale_workspace()
    ms, ok = graph_time(torch, lambda i: fq.fp4_tensor_scale_ws(xs[i % P], cfg, ws, out=tso[i % R]), gr,
                        lambda: same((tso[Lo], fq.fp4_tensor_scale(xs[L], cfg))))
    r["tensor_scale_one_launch_graph"] = dict(report(ms, 2 * n, n, ceiling), replays_match_eager=ok)

    def ts_rtn(i, one_launch):
        if one_launch:
            fq.fp4_tensor_scale_ws(xs[i % P], cfg, ws, out=tso[i % R])
        else:
            fq.fp4_tensor_scale(xs[i % P], cfg, out=tso[i % R])
        fq.fp4_quantize(xs[i % P], cfg, tso[i % R], codes=oc[i % R], scales=os_[i % R])

    def ts_rtn_check():
        t = fq.fp4_tensor_scale(xs[L], cfg)
        return same((tso[Lo], t), *zip((oc[Lo], os_[Lo]), fq.fp4_quantize(xs[L], cfg, t)))
    ms, ok = graph_time(torch, lambda i: ts_rtn(i, True), gr, ts_rtn_check)
    r["tensor_scale_plus_rtn_graph"] = dict(report(ms, 2.5625 * n, n, ceiling), replays_match_eager=ok,
                                            launches=2)
    ms, ok = graph_time(torch, lambda i: ts_rtn(i, False), gr, ts_rtn_check)
    r["tensor_scale_three_launches_plus_rtn_graph"] = dict(report(ms, 2.5625 * n, n, ceiling),
                                                           replays_match_eager=ok, launches=4)
    # both in one launch (fp4_quantize_with_tensor_scale): each workgroup reduces the maximum of its
    # own chunk, waits for s_t and quantizes the chunk it has just read, so x comes from HBM once
    fq.fp4_quantize_with_tensor_scale(xs[0], cfg, ws, ts=tso[0], codes=oc[0], scales=os_[0])
    fused_launches = fq.last_launches
    ms, ok = graph_time(torch, lambda i: fq.fp4_quantize_with_tensor_scale(xs[i % P], cfg, ws, ts=tso[i % R],
                                                                           codes=oc[i % R], scales=os_[i % R]),
                        gr, ts_rtn_check)
    r["tensor_scale_and_rtn_one_launch_graph"] = dict(report(ms, 2.5625 * n, n, ceiling), replays_match_eager=ok,
                                                      launches=fused_launches)
    # supplementary: sixteen tensors of this shape (the 32 input copies in two sets) quantized by one
    # grouped launch, which pays the launch and ramp once for 16 x 16 MiB; checked against single-tensor
    # launches first.  Not the single-tensor workload above, whose figures stand as measured.
    G = 16
    gouts = [[(oc[(G * k + t) % R], os_[(G * k + t) % R]) for t in range(G)] for k in range(R // G)]
    fq.fp4_quantize_grouped(xs[:G], cfg, tss[:G], outs=gouts[0])
    gok = all(torch.equal(a, b) for t in range(G) for a, b in zip(gouts[0][t], fq.fp4_quantize(xs[t], cfg, tss[t])))
    ms = back_to_back(torch, lambda i: fq.fp4_quantize_grouped(xs[G * (i % 2):G * (i % 2) + G], cfg,
                                                               tss[G * (i % 2):G * (i % 2) + G],
                                                               outs=gouts[i % (R // G)]), it)
    r["quantize_rtn_16_tensors_grouped"] = dict(report(ms, 2.5625 * n * G, n * G, ceiling), tensors=G,
                                                grouped_matches_single=bool(gok))
    return r


def wl_c3(args, fq, torch, W, ceiling):
    """KV cache: K and V each (131072*8) x 128, NVFP4 along head_dim; K and V in one grouped launch."""
    it = args.config_iters
    u8 = _u8(torch)
    cfg = fq.Fp4Config()
    rows, cols = W.c3_shape()
    n = rows * cols
    log("KV cache 131072 tokens ...")
    K, V = to_dev(W.c3_kv(0)), to_dev(W.c3_kv(1))
    tk, tv = fq.fp4_tensor_scale(K, cfg), fq.fp4_tensor_scale(V, cfg)
    R = 4   # output sets rotate (4 x 144 MiB), so that the Infinity Cache cannot absorb the writes
    kv_outs = [[(u8(n // 2), u8(n // 16)), (u8(n // 2), u8(n // 16))] for _ in range(R)]
    kv_out = kv_outs[0]
    kds = [torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    vds = [torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    # the grouped launch once, checked against single-tensor launches before it is timed
    fq.fp4_quantize_grouped([K, V], cfg, [tk, tv], outs=kv_out)
    single = [fq.fp4_quantize(K, cfg, tk), fq.fp4_quantize(V, cfg, tv)]
    r = {"grouped_matches_single": all(torch.equal(a, b) for o, s_ in zip(kv_out, single) for a, b in zip(o, s_))}
    del single
    r["quantize_kv_grouped"] = report(back_to_back(torch, lambda i: fq.fp4_quantize_grouped([K, V], cfg, [tk, tv], outs=kv_outs[i % R]), it), 2 * 2.5625 * n, 2 * n, ceiling)

    def deq(i):
        o = kv_outs[i % R]
        fq.fp4_dequantize(o[0][0], o[0][1], cfg, rows, cols, tk, out=kds[i % 2])
        fq.fp4_dequantize(o[1][0], o[1][1], cfg, rows, cols, tv, out=vds[i % 2])
    r["dequantize_kv_bf16"] = report(back_to_back(torch, deq, it), 2 * 2.5625 * n, 2 * n, ceiling)
    del kv_outs, kds, vds
    return r


def wl_c4(args, fq, torch, W, ceiling):
    """One deep guidance-cache layer: 8 expert slices 4096x1536 + activations 8192x4096, grouped."""
    it = args.config_iters
    u8 = _u8(torch)
    cfg = fq.Fp4Config()
    log("guidance-cache layer ...")
    xs, xrs, shapes = [], [], []
    for name, rr, cc, sigma, seed, stream in W.c4_tensors(20):
        xh, xrh = W.c4_pair(rr, cc, sigma, seed, stream)
        xs.append(to_dev(xh))
        xrs.append(to_dev(xrh))
        shapes.append((rr, cc))
    n_layer = sum(rr * cc for rr, cc in shapes)
    tss = [fq.fp4_tensor_scale(x, cfg) for x in xrs]
    roll = [(u8(rr * cc // 2), u8(rr * cc // 16), u8(rr * cc // 8)) for rr, cc in shapes]
    tr = [(u8(rr * cc // 2), u8(rr * cc // 16)) for rr, cc in shapes]
    fq.fp4_quantize_grouped(xrs, cfg, tss, emit=True, outs=roll)
    guides = [(o[2], o[1]) for o in roll]
    pk = [(u8(rr * cc // 8), u8(rr * cc // 16)) for rr, cc in shapes]

    def pack(i):
        for (rr, cc), o, p in zip(shapes, roll, pk):
            fq.guide_pack(o[0], o[1], cfg, rr, cc, bits=p[0], gscales=p[1])
    # each grouped launch once, checked against single-tensor launches before it is timed
    ok = True
    fq.fp4_quantize_grouped(xs, cfg, tss, guides=guides, outs=tr)
    fq.guide_pack_grouped([(o[0], o[1], rr, cc) for (rr, cc), o in zip(shapes, roll)], cfg, outs=pk)
    for t in range(len(shapes)):
        rr, cc = shapes[t]
        ok = ok and all(torch.equal(a, b) for a, b in zip(roll[t], fq.fp4_quantize(xrs[t], cfg, tss[t], emit=True)))
        ok = ok and all(torch.equal(a, b) for a, b in zip(tr[t], fq.fp4_quantize_guided(xs[t], cfg, *guides[t], tss[t])))
        ok = ok and all(torch.equal(a, b) for a, b in zip(pk[t], fq.guide_pack(roll[t][0], roll[t][1], cfg, rr, cc)))
    r = {"grouped_matches_single": bool(ok)}
    # the trainer's tensors against the rollout's codes, summed over the layer's nine tensors
    mm = [mismatch_counts(fq, xs[t], cfg, roll[t][0], roll[t][1], tss[t]) for t in range(len(shapes))]
    tot = {k: sum(m[k] for m in mm) for k in ("elements", "non_adjacent", "mismatched", "rtn_differs")}
    r["guide_mismatch_counts"] = dict(tot, **{k + "_frac": tot[k] / tot["elements"]
                                              for k in ("non_adjacent", "mismatched", "rtn_differs")})
    # timing: the layer's inputs in two copies (2 x 160 MiB per side) and outputs in four sets, so that the
    # Infinity Cache serves neither the reads nor the writes
    R = 4
    xs2 = [xs, [torch.roll(x, 7, 0) for x in xs]]
    xrs2 = [xrs, [torch.roll(x, 7, 0) for x in xrs]]
    rolls = [roll] + [[(u8(rr * cc // 2), u8(rr * cc // 16), u8(rr * cc // 8)) for rr, cc in shapes] for _ in range(R - 1)]
    trs = [tr] + [[(u8(rr * cc // 2), u8(rr * cc // 16)) for rr, cc in shapes] for _ in range(R - 1)]
    for k in range(1, R):
        fq.fp4_quantize_grouped(xrs2[k % 2], cfg, tss, emit=True, outs=rolls[k])
    gds = [[(o[2], o[1]) for o in rl] for rl in rolls]
    r["rollout_rtn_emit_grouped"] = report(back_to_back(torch, lambda i: fq.fp4_quantize_grouped(xrs2[i % 2], cfg, tss, emit=True, outs=rolls[i % R]), it), 2.6875 * n_layer, n_layer, ceiling)
    r["trainer_guided_grouped"] = report(back_to_back(torch, lambda i: fq.fp4_quantize_grouped(xs2[i % 2], cfg, tss, guides=gds[i % R], outs=trs[i % R]), it), 2.75 * n_layer, n_layer, ceiling)
    # guide_pack reads the rollout codes (47 MB per set) and writes 16 MB: eight sets of both
    G = 8
    codes_sets = rolls + [[(o[0].clone(), o[1].clone()) for o in rolls[k % R]] for k in range(R, G)]
    pks = [pk] + [[(u8(rr * cc // 8), u8(rr * cc // 16)) for rr, cc in shapes] for _ in range(G - 1)]

    def pack(i):
        for (rr, cc), o, p in zip(shapes, codes_sets[i % G], pks[i % G]):
            fq.guide_pack(o[0], o[1], cfg, rr, cc, bits=p[0], gscales=p[1])
    r["guide_pack_9_launches"] = report(back_to_back(torch, pack, it), 0.75 * n_layer, n_layer, ceiling)
    # the same nine tensors in one launch (argument arrays built once, so the host stays ahead)
    garrs = [(fq._CGuide * len(shapes))(*[fq._CGuide(o[0].data_ptr(), o[1].data_ptr(), rr, cc, q[0].data_ptr(),
                                                     q[1].data_ptr()) for (rr, cc), o, q in
                                          zip(shapes, codes_sets[k], pks[k])]) for k in range(G)]
    gcfg = cfg.c()
    gstream = torch.cuda.current_stream().cuda_stream
    import ctypes
    r["guide_pack_grouped"] = report(back_to_back(torch, lambda i: fq.lib().guide_pack_grouped(
        ctypes.byref(gcfg), len(shapes), garrs[i % G], gstream), it), 0.75 * n_layer, n_layer, ceiling)
    del xs2, xrs2, rolls, trs, codes_sets, pks
    per_layer_guide = n_layer // 8 + n_layer // 16
    per_layer_full = n_layer // 2 + n_layer // 16
    r["cache_bytes_20_deep_layers"] = per_layer_guide * 20
    r["full_codes_scales_40_layers"] = per_layer_full * 40
    r["cache_ratio"] = round(per_layer_guide * 20 / (per_layer_full * 40), 6)
    return r


def wl_c5(args, fq, torch, W, ceiling):
    """Uniform grid + RHT16 + SR on a 65536x8192 GEMM operand (1 GiB)."""
    it = args.config_iters
    u8 = _u8(torch)
    rows, cols = W.c5_shape()
    n = rows * cols
    log("uniform + RHT16 + SR 65536x8192 (generating 1 GiB) ...")
    x = to_dev(W.c5_x(rows, cols))
    # the quantized operand (288 MB, more than the 256 MB Infinity Cache holds) waits for its product:
    # its stores stream past the caches (stream_out)
    cfg5 = fq.Fp4Config(grid=fq.UNIFORM, rounding=fq.SR, rht16=True, rht_seed=W.C5_RHT_SEED, sr_seed=W.C5_SR_SEED,
                        stream_out=True)
    ts = fq.fp4_tensor_scale(x, cfg5)
    outs5 = [(u8(n // 2), u8(n // 16)) for _ in range(2)]   # 2 x 288 MB: the writes cannot stay in the cache
    tso = torch.empty(1, dtype=torch.float32, device="cuda")
    k5 = max(5, it // 2)
    r = {}
    r["tensor_scale_rht"] = report(back_to_back(torch, lambda i: fq.fp4_tensor_scale(x, cfg5, out=tso), k5), 2 * n, n, ceiling)
    r["quantize_rht_sr_uniform"] = report(back_to_back(torch, lambda i: fq.fp4_quantize(x, cfg5, ts, codes=outs5[i % 2][0], scales=outs5[i % 2][1]), k5), 2.5625 * n, n, ceiling)
    return r


# --workload name -> (key under "workloads", function)
WORKLOADS = {
    "c1": ("nvfp4_act_4096x2048", wl_c1),
    "c3": ("nvfp4_kv_131072x8x128", wl_c3),
    "c4": ("guide_cache_layer_8x4096x1536_plus_8192x4096", wl_c4),
    "c5": ("uniform_rht16_sr_65536x8192", wl_c5),
}


def other_workloads(args, fq, torch, W, ceiling, names=("c1", "c3", "c4", "c5")):
    res = {}
    for name in names:
        key, fn = WORKLOADS[name]
        res[key] = fn(args, fq, torch, W, ceiling)
        torch.cuda.empty_cache()
    return res


# the main kernel of each workload, whose roofline a single-workload run reports
ROOFLINE_KERNEL = {
    "c1": "tensor_scale_and_rtn_one_launch_graph",
    "c3": "quantize_kv_grouped",
    "c4": "trainer_guided_grouped",
    "c5": "quantize_rht_sr_uniform",
}


def workload_roofline(name, r, sha):
    """HBM roofline entry of a workload's main kernel (back-to-back or graph launch duration)."""
    if not r or name not in ROOFLINE_KERNEL:
        return None
    k = ROOFLINE_KERNEL[name]
    e = r[k]
    return {"bound": "hbm", "kernel": k, "achieved": e["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(e["GBps"] / PEAK_HBM_GBS, 4), "traffic": read_traffic(f"{k}@{name}", sha),
            "algorithmic_bytes_per_launch": e["bytes"], "avg_launch_us": e["us"]}


def gemm_workload(args, fq, torch, W):
    """MXFP4 product C = A * B^T: A the activations [8192, 4096] N(0, 1), B one expert weight
    [1536 out, 4096 in] N(0, 0.02^2) (the guidance-cache layer's tensors, weight stored out x in so
    that both operands are blocked along K), both quantized by fp4_quantize (MXFP4, RTN)."""
    M, N, K = W.GEMM_SHAPE
    log(f"MXFP4 GEMM {M}x{N}x{K} ...")
    xa = to_dev(W.f32_to_bf16_rne(W.normal_outliers_f32(M, K, 1020, 16, 0.0, 1.0)))
    xb = to_dev(W.f32_to_bf16_rne(W.normal_outliers_f32(N, K, 1020, 0, 0.0, 1.0, sigma=0.02)))
    cfg = fq.Fp4Config(format=fq.MXFP4)
    a, asc = fq.fp4_quantize(xa, cfg)
    b, bsc = fq.fp4_quantize(xb, cfg)
    del xa, xb
    flops = 2.0 * M * N * K
    reps = max(20, args.config_iters)
    res = {"M": M, "N": N, "K": K, "flops": flops}
    for name, dt in (("bf16_out", torch.bfloat16), ("f32_out", torch.float32)):
        out = torch.empty((M, N), dtype=dt, device="cuda")
        ms = back_to_back(torch, lambda i: fq.fp4_gemm_mxfp4(a, asc, b, bsc, M, N, K, out=out), reps, warm=5)
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
                     "us_p10_median_p90_single_launch": take_spread()}
    # the same weight shape as 8 routed experts of 1024 tokens each, in one grouped launch
    E = 8
    ws = [fq.fp4_quantize(to_dev(W.f32_to_bf16_rne(W.normal_outliers_f32(N, K, 1020, 2 * e, 0.0, 1.0, sigma=0.02))),
                          cfg) for e in range(E)]
    rows = M // E
    prods = [(a[e * rows * K // 2:(e + 1) * rows * K // 2], asc[e * rows * K // 32:(e + 1) * rows * K // 32],
              ws[e][0], ws[e][1], rows, N, K) for e in range(E)]
    outs = fq.fp4_gemm_mxfp4_grouped(prods, dtype=torch.bfloat16)
    # the argument array is built once, so the host keeps ahead of the GPU between launches
    arr = (fq._CGemm * E)(*[fq._CGemm(ac.data_ptr(), asc_.data_ptr(), bc.data_ptr(), bsc_.data_ptr(), m, n, k,
                                      o.data_ptr(), n) for (ac, asc_, bc, bsc_, m, n, k), o in zip(prods, outs)])
    stream = torch.cuda.current_stream().cuda_stream
    ms = back_to_back(torch, lambda i: fq.lib().fp4_gemm_mxfp4_grouped(E, arr, fq.OUT_BF16, stream), reps, warm=5)
    tf = flops / (ms * 1e-3) / 1e12
    res["grouped_8_experts_bf16_out"] = {"experts": E, "tokens_per_expert": rows, "us": round(ms * 1e3, 2),
                                         "TFLOPs": round(tf, 1), "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
                                         "us_p10_median_p90_single_launch": take_spread()}
    # producer-side fusion: the product's epilogue writes the MXFP4 codes, scales and guide bits of the
    # bf16-rounded C (the next layer's quantized input and the rollout's guide) instead of C; against the
    # plain product with bf16 output followed by fp4_quantize with emission
    qc, qs, qb = (torch.empty(M * N // d, dtype=torch.uint8, device="cuda") for d in (2, 32, 8))
    cb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    fq.fp4_gemm_mxfp4_quantize(a, asc, b, bsc, M, N, K, codes=qc, scales=qs, bits=qb)
    ref = fq.fp4_quantize(fq.fp4_gemm_mxfp4(a, asc, b, bsc, M, N, K, out=cb), cfg, emit=True)
    same = all(torch.equal(x, y) for x, y in zip((qc, qs, qb), ref))
    ms_f = back_to_back(torch, lambda i: fq.fp4_gemm_mxfp4_quantize(a, asc, b, bsc, M, N, K, codes=qc, scales=qs,
                                                                    bits=qb), reps, warm=5)
    sp_f = take_spread()

    def two_step(i):
        fq.fp4_gemm_mxfp4(a, asc, b, bsc, M, N, K, out=cb)
        fq.fp4_quantize(cb, cfg, emit=True, codes=qc, scales=qs, bits=qb)
    ms_2 = back_to_back(torch, two_step, reps, warm=5)
    res["fused_quantize_epilogue"] = {
        "us": round(ms_f * 1e3, 2), "TFLOPs": round(flops / (ms_f * 1e-3) / 1e12, 1),
        "us_p10_median_p90_single_launch": sp_f,
        "us_product_bf16_then_quantize_emit": round(ms_2 * 1e3, 2),
        "speedup_vs_two_launches": round(ms_2 / ms_f, 3),
        "equals_product_then_quantize": bool(same),
        "bytes_written": M * N // 2 + M * N // 32 + M * N // 8, "bytes_of_bf16_c_not_written": 2 * M * N}
    # the same with the result stored as NVFP4 under a given tensor scale (a KV-cache write), against the
    # plain product followed by fp4_quantize (NVFP4, RTN, emission) with that scale
    nv = fq.Fp4Config()
    ts = fq.fp4_tensor_scale(cb, nv)
    ns_ = torch.empty(M * N // 16, dtype=torch.uint8, device="cuda")
    fq.fp4_gemm_mxfp4_quantize_nvfp4(a, asc, b, bsc, M, N, K, ts, codes=qc, scales=ns_, bits=qb)
    ref = fq.fp4_quantize(cb, nv, ts, emit=True)
    same_nv = all(torch.equal(x, y) for x, y in zip((qc, ns_, qb), ref))
    ms_fn = back_to_back(torch, lambda i: fq.fp4_gemm_mxfp4_quantize_nvfp4(a, asc, b, bsc, M, N, K, ts, codes=qc,
                                                                          scales=ns_, bits=qb), reps, warm=5)
    sp_fn = take_spread()

    def two_step_nv(i):
        fq.fp4_gemm_mxfp4(a, asc, b, bsc, M, N, K, out=cb)
        fq.fp4_quantize(cb, nv, ts, emit=True, codes=qc, scales=ns_, bits=qb)
    ms_2n = back_to_back(torch, two_step_nv, reps, warm=5)
    res["fused_quantize_epilogue_nvfp4"] = {
        "us": round(ms_fn * 1e3, 2), "TFLOPs": round(flops / (ms_fn * 1e-3) / 1e12, 1),
        "us_p10_median_p90_single_launch": sp_fn,
        "us_product_bf16_then_quantize_emit": round(ms_2n * 1e3, 2),
        "speedup_vs_two_launches": round(ms_2n / ms_fn, 3),
        "equals_product_then_quantize": bool(same_nv),
        "bytes_written": M * N // 2 + M * N // 16 + M * N // 8, "bytes_of_bf16_c_not_written": 2 * M * N}
    del qc, qs, qb, cb, ref, outs, ws, prods, arr, ns_, ts
    # a square product, 16384^3 with bf16 out (256 x 256 tiles, 16 rounds): random E2M1 codes and
    # E8M0 scales 120..130, drawn on the device
    S = 16384
    g = torch.Generator(device="cuda").manual_seed(3)
    sa_ = torch.randint(0, 256, (S * S // 2,), dtype=torch.uint8, device="cuda", generator=g)
    sas = torch.randint(120, 131, (S * S // 32,), dtype=torch.uint8, device="cuda", generator=g)
    sb_ = torch.randint(0, 256, (S * S // 2,), dtype=torch.uint8, device="cuda", generator=g)
    sbs = torch.randint(120, 131, (S * S // 32,), dtype=torch.uint8, device="cuda", generator=g)
    sc = torch.empty((S, S), dtype=torch.bfloat16, device="cuda")
    ms = back_to_back(torch, lambda i: fq.fp4_gemm_mxfp4(sa_, sas, sb_, sbs, S, S, S, out=sc), max(5, reps // 4), warm=2)
    tf = 2.0 * S ** 3 / (ms * 1e-3) / 1e12
    res["square_16384_bf16_out"] = {"M": S, "N": S, "K": S, "us": round(ms * 1e3, 2), "TFLOPs": round(tf, 1),
                                    "frac_fp4_peak": round(tf / PEAK_FP4_TFLOPS, 4),
                                    "us_p10_median_p90_single_launch": take_spread()}
    del sa_, sas, sb_, sbs, sc
    r = res["bf16_out"]
    res["roofline"] = {"bound": "mfma", "kernel": "k_gemm_mx_lds", "achieved": r["TFLOPs"], "peak": PEAK_FP4_TFLOPS,
                       "unit": "TFLOP/s", "frac": r["frac_fp4_peak"], "traffic": None,
                       "algorithmic_flops_per_launch": flops, "avg_launch_us": r["us"]}
    return res


def main():
    global SETTLE_MS
    args = parse()
    SETTLE_MS = args.settle_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); runs on several GPUs are not "
              "part of this path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from precision_rl_amd import fp4q as fq, workloads as W
    fq.lib()
    torch.cuda.set_device(0)
    if args.gemm_only:
        args.workload = "gemm"
    if args.workload in WORKLOADS:
        ceiling = copy_ceiling(torch, fq)
        key, fn = WORKLOADS[args.workload]
        r = fn(args, fq, torch, W, ceiling["GBps"])
        line = {"metric": f"{key} kernels", "workload": key, "n_gpus": 1, "data": "synthetic",
                "copy_ceiling": ceiling, "results": r, "source_sha": source_sha()}
        rl = workload_roofline(args.workload, r, source_sha())
        if rl:
            line["roofline"] = rl
        print(json.dumps(line), flush=True)
        return
    if args.workload == "gemm":
        g = gemm_workload(args, fq, torch, W)
        print(json.dumps({"metric": "MXFP4 GEMM TFLOP/s", "value": g["bf16_out"]["TFLOPs"], "unit": "TFLOP/s",
                          "n_gpus": 1, "higher_is_better": True, "dtype": "fp4 x fp4 -> f32 (bf16 out)",
                          "data": "synthetic", "config": {"workload": "MXFP4 GEMM activations [8192, 4096] x "
                                                                     "expert weight [1536, 4096]^T"},
                          "roofline": g["roofline"], "gemm": g}), flush=True)
        return

    ceiling = copy_ceiling(torch, fq)
    h = headline(args, fq, torch, W, ceiling["GBps"])
    import oracle as oracle_mod  # CPU baseline and the parity sample only
    parity = parity_sample(torch, h, oracle_mod)
    if not parity:
        log("PARITY FAILURE on the headline sample")
    cpu = cpu_all = None
    if not (args.quick or args.no_cpu_baseline):
        log("CPU baseline (oracle) ...")
        cpu = cpu_baseline(args, W, oracle_mod, h)
        # the same sample on all host threads of one GPU's share (at most 16)
        cpu_all = cpu_baseline(args, W, oracle_mod, h, threads=max(1, min(16, os.cpu_count() or 1)))
    workloads = {} if args.quick else other_workloads(args, fq, torch, W, ceiling["GBps"])
    if not args.quick:
        workloads["mxfp4_gemm_8192x1536x4096"] = gemm_workload(args, fq, torch, W)

    n = h["n"]
    value = h["step_bytes"] / (h["ms_step"] * 1e-3) / 1e9
    # the kernel with the largest share of the step, by its back-to-back duration (the figure rocprofv3's
    # kernel trace reports; the in-step per-launch events include the event overhead)
    dom = max(h["kernels"], key=lambda k: h["kernels"][k]["us_back_to_back"])
    dk = h["kernels"][dom]
    ach = dk["GBps_back_to_back"]
    sha = source_sha()
    out = {
        "metric": "FP4 quantize GB/s and Gelem/s (RTN & guided) as % of MI355X HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_step"], 4),
        "ms_per_step_serial": round(h["ms_serial"], 4),
        "ms_per_step_two_streams": round(h["ms_two"], 4),
        "streams": args.streams,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "MXFP4 MoE expert activations 16384x4096 bf16 Student-t(4): rollout RTN "
                               "quantize + guide_pack, trainer guided quantize, dequantize to bf16, SR "
                               "quantize (Philox key 1) of the previous batch",
                   "streams": args.streams,
                   "rows": h["rows"], "cols": h["cols"], "block": 32, "scale": "E8M0",
                   "elements_per_kernel": n, "bytes_per_step": int(h["step_bytes"])},
        "gelem_per_s": round(5 * n / (h["ms_step"] * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(value / PEAK_HBM_GBS, 4),
        "frac_copy_ceiling": round(value / ceiling["GBps"], 4),
        "parity_sample_ok": parity,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": read_traffic(f"{dom}@c2", sha),
                     "algorithmic_bytes_per_launch": dk["bytes"], "avg_launch_us": dk["us_back_to_back"],
                     "median_launch_us_in_step": dk["us"]},
        "roofline_c5": workload_roofline("c5", workloads.get(WORKLOADS["c5"][0]), sha),
        "cpu_baseline": cpu,
        "cpu_baseline_all_threads": cpu_all,
        "step_us_p10_median_p90": h["step_us_p10_median_p90"],
        "copy_ceiling": ceiling,
        "kernels": h["kernels"],
        "fake_quantize_guided_bf16": h["fake"],
        "guide_mismatch_c2": h["diag"],
        "workloads": workloads,
        "source_sha": sha,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
