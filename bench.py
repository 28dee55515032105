#!/usr/bin/env python3
"""Throughput of the block-scaled FP4 quantization path on one MI355X.

Headline workload (one "step" = one pass of the hot path over one batch):
MXFP4 quantization of MoE expert activations, 16384 tokens x 4096 hidden,
bf16 Student-t(4) values, 32-element blocks with E8M0 scales:
  1. rollout side: RTN quantize of the rollout copy x_r,
  2. guide_pack of its codes and scales (1 mantissa bit + block scale),
  3. trainer side: guided quantize of x with that guide,
  4. stochastic rounding (Philox, key 1) of an activation batch of the same
     shape (the previous batch's x, so no input is re-read from the last-level
     cache within a step),
  5. dequantize of the guided codes to bf16.
``value`` = algorithmic bytes of the step / step time, in GB/s.  Inputs are
resident in HBM before timing; a rotating pool of input sets (>= 768 MiB)
keeps the 256 MB Infinity Cache from serving re-reads across steps.

The other workloads (NVFP4 activation 4096x2048 with RTN/guided, the KV cache
at 131072 tokens, one deep guidance-cache layer, the uniform grid with RHT16
and SR on a 65536x8192 GEMM operand) are timed after it and reported under
"workloads".  Per-kernel durations come from HIP events recorded on the
stream the kernels run on.  The CPU baseline is the oracle timed on a
bounded row sample of the headline step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
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


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline workload only, no CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="rows of the CPU-baseline sample")
    ap.add_argument("--config-iters", type=int, default=20)
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
        tot, cnt = {}, {}
        for name, s, e in self.events:
            tot[name] = tot.get(name, 0.0) + s.elapsed_time(e)
            cnt[name] = cnt.get(name, 0) + 1
        return {k: (tot[k] / cnt[k], cnt[k]) for k in tot}


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


# ---------------------------------------------------------------- headline step
def headline(args, fq, torch, W):
    rows, cols = W.c2_shape()
    n = rows * cols
    log(f"generating C2 {rows}x{cols} Student-t(4) ...")
    x_h, xr_h = W.c2_pair(rows, cols, seed=1)
    cfg_rtn = fq.Fp4Config(format=fq.MXFP4)
    cfg_sr = fq.Fp4Config(format=fq.MXFP4, rounding=fq.SR, sr_seed=W.C2_SR_SEED)
    P = 3  # rotating input sets: 3 x 256 MiB
    x0, xr0 = to_dev(x_h), to_dev(xr_h)
    xs = [x0] + [torch.roll(x0, shifts=(s * 977), dims=0) for s in range(1, P)]
    xrs = [xr0] + [torch.roll(xr0, shifts=(s * 977), dims=0) for s in range(1, P)]
    B = 32
    u8 = lambda k: torch.empty(k, dtype=torch.uint8, device="cuda")
    outs = [dict(rc=u8(n // 2), rs=u8(n // B), gb=u8(n // 8), gs=u8(n // B), gc=u8(n // 2), gsc=u8(n // B),
                 sc=u8(n // 2), ss=u8(n // B), dq=torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda"))
            for _ in range(P)]

    def step_fns(k):
        s = k % P
        o = outs[s]
        return {
            "quantize_rtn": lambda: fq.fp4_quantize(xrs[s], cfg_rtn, None, codes=o["rc"], scales=o["rs"]),
            "guide_pack": lambda: fq.guide_pack(o["rc"], o["rs"], cfg_rtn, rows, cols, bits=o["gb"], gscales=o["gs"]),
            "quantize_guided": lambda: fq.fp4_quantize_guided(xs[s], cfg_rtn, o["gb"], o["gs"], None,
                                                              codes=o["gc"], scales=o["gsc"]),
            "quantize_sr": lambda: fq.fp4_quantize(xs[(s + 2) % P], cfg_sr, None, codes=o["sc"], scales=o["ss"]),
            "dequantize_bf16": lambda: fq.fp4_dequantize(o["gc"], o["gsc"], cfg_rtn, rows, cols, None, out=o["dq"]),
        }

    def one(fn):
        fn()

    def step(k, timer=None):
        for name, fn in step_fns(k).items():
            if timer:
                timer.run(name, fn)
            else:
                fn()

    bytes_per = {  # algorithmic bytes per element of each kernel (MXFP4, B = 32)
        "quantize_rtn": 2 + 0.5 + 1 / 32,
        "guide_pack": 0.5 + 1 / 32 + 1 / 8 + 1 / 32,
        "quantize_guided": 2 + 1 / 8 + 1 / 32 + 0.5 + 1 / 32,
        "quantize_sr": 2 + 0.5 + 1 / 32,
        "dequantize_bf16": 0.5 + 1 / 32 + 2,
    }
    step_bytes = sum(bytes_per.values()) * n

    log("warmup ...")
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # timed region 1: whole steps, no per-kernel events
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for k in range(args.steps):
        step(k)
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / args.steps
    # timed region 2: the same steps with events around every kernel
    timer = KernelTimer()
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(k, timer)
    torch.cuda.synchronize()
    ks = timer.summary()
    kernels = {}
    for name, (ms, cnt) in ks.items():
        b = bytes_per[name] * n
        kernels[name] = {"us": round(ms * 1e3, 2), "launches": cnt, "bytes": int(b),
                         "GBps": round(b / (ms * 1e-3) / 1e9, 1), "Gelem_per_s": round(n / (ms * 1e-3) / 1e9, 1),
                         "frac_hbm_peak": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    # back-to-back launches of each kernel alone (events around the loop): the average
    # launch duration used for the roofline, comparable with rocprofv3's kernel durations
    single = {}
    for name in kernels:
        t_a = torch.cuda.Event(enable_timing=True)
        t_b = torch.cuda.Event(enable_timing=True)
        reps = args.steps
        for k in range(2):
            one(step_fns(k)[name])
        torch.cuda.synchronize()
        t_a.record()
        for k in range(reps):
            step_fns(k)[name]()
        t_b.record()
        torch.cuda.synchronize()
        single[name] = t_a.elapsed_time(t_b) / reps
    for name, ms in single.items():
        b = bytes_per[name] * n
        kernels[name]["us_back_to_back"] = round(ms * 1e3, 2)
        kernels[name]["GBps_back_to_back"] = round(b / (ms * 1e-3) / 1e9, 1)
    return dict(rows=rows, cols=cols, n=n, ms_step=ms_step, wall=wall, step_bytes=step_bytes,
                kernels=kernels, bytes_per=bytes_per, x_h=x_h, xr_h=xr_h, outs=outs[0], cfg_rtn=cfg_rtn,
                cfg_sr=cfg_sr, xs=xs)


def copy_ceiling(torch, mib=256, iters=20):
    """A plain streaming read+write of known size (torch's vectorized elementwise kernel,
    y = -x in fp32): the practical streaming ceiling next to the quantize kernels."""
    n = mib * (1 << 20) // 4
    bufs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(4)]
    for b in bufs:
        b.fill_(1.0)
    timer = KernelTimer()
    for i in range(iters):
        timer.run("copy", lambda: torch.neg(bufs[(2 * i) % 4], out=bufs[(2 * i + 1) % 4]))
    torch.cuda.synchronize()
    ms = timer.summary()["copy"][0]
    return {"bytes_per_launch": 2 * n * 4, "us": round(ms * 1e3, 2),
            "GBps": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}


def parity_sample(fq, torch, W, h, oracle_mod, rows_s=64):
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


def cpu_baseline(args, W, oracle_mod, h):
    """The oracle (unchanged) on rows [0, R) of the headline step, one host thread."""
    O = oracle_mod
    R = min(args.cpu_rows, h["rows"])
    cols = h["cols"]
    x, xr = h["x_h"][:R], h["xr_h"][:R]
    oc = O.Cfg(format=O.MXFP4)
    osr = O.Cfg(format=O.MXFP4, sr_seed=W.C2_SR_SEED)
    t = time.perf_counter()
    rc, rs = O.quantize(oc, O.RTN, xr)
    gb, gs = O.guide_pack(oc, rc, rs, R, cols)
    gc, gsc = O.quantize(oc, O.GUIDED, x, guide_bits=gb, guide_scales=gs)
    O.quantize(osr, O.SR, x)
    O.dequantize(oc, gc, gsc, 1.0, R, cols, out_bf16=True)
    dt = time.perf_counter() - t
    b = sum(h["bytes_per"].values()) * R * cols
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"rows 0..{R} of the 16384x4096 workload ({R * cols} elements), all five kernels "
                      f"of the step, single thread, {dt:.1f} s"}


# ---------------------------------------------------------------- other workloads
def time_loop(torch, fns, iters):
    """Average ms of each named callable over `iters` rounds, events around each call."""
    timer = KernelTimer()
    for name, fn in fns:  # warm
        fn()
    torch.cuda.synchronize()
    for _ in range(iters):
        for name, fn in fns:
            timer.run(name, fn)
    torch.cuda.synchronize()
    return {k: v[0] for k, v in timer.summary().items()}


def report(ms, nbytes, n):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 2), "bytes": int(nbytes), "GBps": round(gbs, 1),
            "Gelem_per_s": round(n / (ms * 1e-3) / 1e9, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def other_workloads(args, fq, torch, W):
    res = {}
    it = args.config_iters
    u8 = lambda k: torch.empty(k, dtype=torch.uint8, device="cuda")

    # NVFP4 activation 4096x2048 (16 MiB): a pool of 32 copies keeps it out of the caches
    rows, cols = W.c1_shape()
    n = rows * cols
    log("C1 ...")
    x0, xr0 = to_dev(W.c1_x(rows, cols)), to_dev(W.c1_rollout(rows, cols))
    cfg = fq.Fp4Config()
    P = 32
    xs = [torch.roll(x0, s * 61, 0) for s in range(P)]
    xrs = [torch.roll(xr0, s * 61, 0) for s in range(P)]
    tss = [fq.fp4_tensor_scale(xr, cfg) for xr in xrs]
    guides = [fq.fp4_quantize(xrs[s], cfg, tss[s], emit=True) for s in range(P)]
    oc, os_, ob = u8(n // 2), u8(n // 16), u8(n // 8)
    k = [0]

    def nxt():
        k[0] = (k[0] + 1) % P
        return k[0]
    ms = time_loop(torch, [
        ("tensor_scale", lambda: fq.fp4_tensor_scale(xs[nxt()], cfg, out=tss[k[0]])),
        ("quantize_rtn", lambda: fq.fp4_quantize(xs[nxt()], cfg, tss[k[0]], codes=oc, scales=os_)),
        ("quantize_rtn_emit", lambda: fq.fp4_quantize(xs[nxt()], cfg, tss[k[0]], emit=True, codes=oc, scales=os_, bits=ob)),
        ("quantize_guided", lambda: fq.fp4_quantize_guided(xs[nxt()], cfg, guides[k[0]][2], guides[k[0]][1], tss[k[0]], codes=oc, scales=os_)),
    ], it)
    res["nvfp4_act_4096x2048"] = {
        "tensor_scale": report(ms["tensor_scale"], 2 * n, n),
        "quantize_rtn": report(ms["quantize_rtn"], 2.5625 * n, n),
        "quantize_rtn_emit": report(ms["quantize_rtn_emit"], 2.6875 * n, n),
        "quantize_guided": report(ms["quantize_guided"], 2.75 * n, n),
    }
    del xs, xrs, guides

    # KV cache: K and V each (131072*8) x 128, NVFP4 along head_dim
    rows, cols = W.c3_shape()
    n = rows * cols
    log("C3 ...")
    K, V = to_dev(W.c3_kv(0)), to_dev(W.c3_kv(1))
    tk, tv = fq.fp4_tensor_scale(K, cfg), fq.fp4_tensor_scale(V, cfg)
    kc, ks_, vc, vs = u8(n // 2), u8(n // 16), u8(n // 2), u8(n // 16)
    kd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    vd = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    ms = time_loop(torch, [
        ("quantize_k", lambda: fq.fp4_quantize(K, cfg, tk, codes=kc, scales=ks_)),
        ("quantize_v", lambda: fq.fp4_quantize(V, cfg, tv, codes=vc, scales=vs)),
        ("dequantize_k", lambda: fq.fp4_dequantize(kc, ks_, cfg, rows, cols, tk, out=kd)),
        ("dequantize_v", lambda: fq.fp4_dequantize(vc, vs, cfg, rows, cols, tv, out=vd)),
    ], it)
    res["nvfp4_kv_131072x8x128"] = {
        "quantize_kv": report(ms["quantize_k"] + ms["quantize_v"], 2 * 2.5625 * n, 2 * n),
        "dequantize_kv_bf16": report(ms["dequantize_k"] + ms["dequantize_v"], 2 * 2.5625 * n, 2 * n),
    }
    del K, V, kd, vd

    # one deep guidance-cache layer: 8 experts 4096x1536 + activations 8192x4096
    log("C4 ...")
    tens = []
    for name, r, c, sigma, seed, stream in W.c4_tensors(20):
        xh, xrh = W.c4_pair(r, c, sigma, seed, stream)
        tens.append((to_dev(xh), to_dev(xrh), r, c))
    n_layer = sum(r * c for _, _, r, c in tens)
    bufs = []
    for x, xr, r, c in tens:
        m = r * c
        ts = fq.fp4_tensor_scale(xr, cfg)
        bufs.append(dict(x=x, xr=xr, r=r, c=c, ts=ts, rc=u8(m // 2), rs=u8(m // 16), gb=u8(m // 8),
                         gs=u8(m // 16), gc=u8(m // 2), gsc=u8(m // 16)))

    def rollout():
        for b in bufs:
            fq.fp4_quantize(b["xr"], cfg, b["ts"], codes=b["rc"], scales=b["rs"])

    def pack():
        for b in bufs:
            fq.guide_pack(b["rc"], b["rs"], cfg, b["r"], b["c"], bits=b["gb"], gscales=b["gs"])

    def trainer():
        for b in bufs:
            fq.fp4_quantize_guided(b["x"], cfg, b["gb"], b["gs"], b["ts"], codes=b["gc"], scales=b["gsc"])
    ms = time_loop(torch, [("rollout_rtn", rollout), ("guide_pack", pack), ("trainer_guided", trainer)], it)
    per_layer_guide = n_layer // 8 + n_layer // 16
    per_layer_full = n_layer // 2 + n_layer // 16
    res["guide_cache_layer_8x4096x1536_plus_8192x4096"] = {
        "rollout_rtn": report(ms["rollout_rtn"], 2.5625 * n_layer, n_layer),
        "guide_pack": report(ms["guide_pack"], 0.75 * n_layer, n_layer),
        "trainer_guided": report(ms["trainer_guided"], 2.75 * n_layer, n_layer),
        "cache_bytes_20_deep_layers": per_layer_guide * 20,
        "full_codes_scales_40_layers": per_layer_full * 40,
        "cache_ratio": round(per_layer_guide * 20 / (per_layer_full * 40), 6),
    }
    del tens, bufs

    # uniform grid + RHT16 + SR on a 65536x8192 GEMM operand (1 GiB)
    rows, cols = W.c5_shape()
    n = rows * cols
    log("C5 (generating 1 GiB) ...")
    x = to_dev(W.c5_x(rows, cols))
    cfg5 = fq.Fp4Config(grid=fq.UNIFORM, rounding=fq.SR, rht16=True, rht_seed=W.C5_RHT_SEED, sr_seed=W.C5_SR_SEED)
    ts = fq.fp4_tensor_scale(x, cfg5)
    c5c, c5s = u8(n // 2), u8(n // 16)
    ms = time_loop(torch, [
        ("tensor_scale_rht", lambda: fq.fp4_tensor_scale(x, cfg5, out=ts)),
        ("quantize_rht_sr_uniform", lambda: fq.fp4_quantize(x, cfg5, ts, codes=c5c, scales=c5s)),
    ], max(5, it // 2))
    res["uniform_rht16_sr_65536x8192"] = {
        "tensor_scale_rht": report(ms["tensor_scale_rht"], 2 * n, n),
        "quantize_rht_sr_uniform": report(ms["quantize_rht_sr_uniform"], 2.5625 * n, n),
    }
    del x
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not part "
              "of this path", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    from precision_rl_amd import fp4q as fq, workloads as W
    fq.lib()
    torch.cuda.set_device(0)

    h = headline(args, fq, torch, W)
    ceiling = copy_ceiling(torch)
    for k in h["kernels"].values():
        k["frac_copy_ceiling"] = round(k["GBps"] / ceiling["GBps"], 4)
    import oracle as oracle_mod  # CPU baseline and the parity sample only
    parity = parity_sample(fq, torch, W, h, oracle_mod)
    if not parity:
        log("PARITY FAILURE on the headline sample")
    cpu = None
    if not (args.quick or args.no_cpu_baseline):
        log("CPU baseline (oracle) ...")
        cpu = cpu_baseline(args, W, oracle_mod, h)
    workloads = {} if args.quick else other_workloads(args, fq, torch, W)

    n = h["n"]
    value = h["step_bytes"] / (h["ms_step"] * 1e-3) / 1e9
    dom = max(h["kernels"], key=lambda k: h["kernels"][k]["us_back_to_back"])
    dk = h["kernels"][dom]
    ach = dk["GBps_back_to_back"]
    sha = source_sha()
    traffic = read_traffic(f"{dom}@c2", sha)
    out = {
        "metric": "FP4 quantize GB/s and Gelem/s (RTN & guided) as % of MI355X HBM peak",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "MXFP4 MoE expert activations 16384x4096 bf16 Student-t(4): rollout RTN "
                               "quantize + guide_pack, trainer guided quantize, SR quantize (Philox key 1), "
                               "dequantize to bf16",
                   "rows": h["rows"], "cols": h["cols"], "block": 32, "scale": "E8M0",
                   "elements_per_step": n, "bytes_per_step": int(h["step_bytes"])},
        "gelem_per_s": round(5 * n / (h["ms_step"] * 1e-3) / 1e9, 1),
        "frac_hbm_peak": round(value / PEAK_HBM_GBS, 4),
        "parity_sample_ok": parity,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": ach, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": dk["bytes"], "avg_launch_us": dk["us_back_to_back"],
                     "avg_launch_us_in_step": dk["us"]},
        "cpu_baseline": cpu,
        "copy_ceiling": ceiling,
        "kernels": h["kernels"],
        "workloads": workloads,
        "source_sha": sha,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
