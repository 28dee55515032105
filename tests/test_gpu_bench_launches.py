"""Oracle parity of the launches bench.py times, at the size and in the launch
form it times them:

* the grouped K+V quantize of the KV cache (131072 tokens x 8 heads x 128) and
  the dequantization of both to bf16;
* one deep guidance-cache layer (8 expert weights 4096x1536 + activations
  8192x4096): the grouped rollout quantize with guide emission, the grouped
  trainer guided quantize, and the grouped guide_pack of the nine tensors;
* the guided fake quantization of the MoE activations (16384x4096, MXFP4);
* sixteen copies of the NVFP4 activation (4096x2048, rows rotated as bench.py
  rotates them) quantized by one grouped launch under the rollout's tensor scale.

Sampled rows (first, last and random ones) of every output are compared bit for
bit with the oracle.  The oracle's inputs come from the input generators and
from the oracle itself (its own rollout codes make the guide), never from a GPU
output.  Output buffers start as 0xA5 bytes.
"""
import sys
import time

import numpy as np
import pytest
import torch

import oracle as O
from precision_rl_amd import workloads as W

pytestmark = pytest.mark.gpu


def say(*a):
    print("[bench-launches]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from precision_rl_amd import fp4q
    fp4q.lib()
    return fp4q


def dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def poisoned(n):
    return torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")


def sample_rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(k, rows - k), size=k, replace=False)
    return sorted(set(range(k)) | set(range(rows - k, rows)) | set(int(r) for r in mid))


def f32bits(x):
    return np.float32(x).view(np.uint32)


def rows_of(t, r, per_row):
    return t[r * per_row:(r + 1) * per_row].cpu().numpy()


def test_c3_kv_grouped_quantize_and_dequantize(fq):
    rows, cols = W.c3_shape()
    t0 = time.time()
    cfg, oc = fq.Fp4Config(), O.Cfg()
    hs = [W.c3_kv(0), W.c3_kv(1)]
    xs = [dev(h) for h in hs]
    tss = [fq.fp4_tensor_scale(x, cfg) for x in xs]
    o_ts = [O.tensor_scale(oc, h) for h in hs]
    for a, b in zip(tss, o_ts):
        assert f32bits(a.item()) == f32bits(b)
    n = rows * cols
    outs = [(poisoned(n // 2), poisoned(n // 16)) for _ in hs]
    fq.fp4_quantize_grouped(xs, cfg, tss, outs=outs)               # as bench.py times it
    dq = [fq.fp4_dequantize(c, s, cfg, rows, cols, ts) for (c, s), ts in zip(outs, tss)]
    torch.cuda.synchronize()
    for which, h in enumerate(hs):
        idx = sample_rows(rows, 64, seed=30 + which)
        c, s = outs[which]
        for r in idx:
            oc_r, os_r = O.quantize(oc, O.RTN, h[r:r + 1], o_ts[which], row0=r)
            assert (rows_of(c, r, cols // 2) == oc_r).all(), ("codes", which, r)
            assert (rows_of(s, r, cols // 16) == os_r).all(), ("scales", which, r)
            want = O.dequantize(oc, oc_r, os_r, o_ts[which], 1, cols, out_bf16=True)
            assert (dq[which][r].view(torch.int16).cpu().numpy() == want.view(np.int16)).all(), ("dq", which, r)
    say(f"C3 grouped K+V: {2 * len(idx)} rows bit-exact ({time.time() - t0:.1f} s)")


def test_c4_layer_grouped_rollout_trainer_and_guide_pack(fq):
    t0 = time.time()
    cfg, oc = fq.Fp4Config(), O.Cfg()
    tensors = list(W.c4_tensors(20))
    hx, hxr, xs, xrs, shapes = [], [], [], [], []
    for name, r, c, sigma, seed, stream in tensors:
        xh, xrh = W.c4_pair(r, c, sigma, seed, stream)
        hx.append(xh)
        hxr.append(xrh)
        xs.append(dev(xh))
        xrs.append(dev(xrh))
        shapes.append((r, c))
    tss = [fq.fp4_tensor_scale(x, cfg) for x in xrs]
    o_ts = [O.tensor_scale(oc, h) for h in hxr]
    for a, b in zip(tss, o_ts):
        assert f32bits(a.item()) == f32bits(b)
    # the launches bench.py times, in its order
    roll = [(poisoned(r * c // 2), poisoned(r * c // 16), poisoned(r * c // 8)) for r, c in shapes]
    fq.fp4_quantize_grouped(xrs, cfg, tss, emit=True, outs=roll)
    guides = [(o[2], o[1]) for o in roll]
    tr = [(poisoned(r * c // 2), poisoned(r * c // 16)) for r, c in shapes]
    fq.fp4_quantize_grouped(xs, cfg, tss, guides=guides, outs=tr)
    pk = [(poisoned(r * c // 8), poisoned(r * c // 16)) for r, c in shapes]
    fq.guide_pack_grouped([(o[0], o[1], r, c) for (r, c), o in zip(shapes, roll)], cfg, outs=pk)
    torch.cuda.synchronize()
    checked = 0
    for t, (name, r_, c_, *_rest) in enumerate(tensors):
        rows, cols = shapes[t]
        for r in sample_rows(rows, 8, seed=40 + t):
            rc, rs, rb = O.quantize(oc, O.RTN, hxr[t][r:r + 1], o_ts[t], row0=r, emit=True)
            assert (rows_of(roll[t][0], r, cols // 2) == rc).all(), (name, "rollout codes", r)
            assert (rows_of(roll[t][1], r, cols // 16) == rs).all(), (name, "rollout scales", r)
            assert (rows_of(roll[t][2], r, cols // 8) == rb).all(), (name, "emitted bits", r)
            gb, gs = O.guide_pack(oc, rc, rs, 1, cols)
            assert (rows_of(pk[t][0], r, cols // 8) == gb).all(), (name, "guide_pack bits", r)
            assert (rows_of(pk[t][1], r, cols // 16) == gs).all(), (name, "guide_pack scales", r)
            gc, gsc = O.quantize(oc, O.GUIDED, hx[t][r:r + 1], o_ts[t], row0=r, guide_bits=gb, guide_scales=gs)
            assert (rows_of(tr[t][0], r, cols // 2) == gc).all(), (name, "guided codes", r)
            assert (rows_of(tr[t][1], r, cols // 16) == gsc).all(), (name, "guided scales", r)
            checked += 1
    say(f"C4 layer: {checked} rows of 9 tensors bit-exact in 3 grouped launches ({time.time() - t0:.1f} s)")


def test_c2_guided_fake_quantize(fq):
    rows, cols = W.c2_shape()
    t0 = time.time()
    x_h, xr_h = W.c2_pair(rows, cols, seed=1)
    cfg, oc = fq.Fp4Config(format=fq.MXFP4), O.Cfg(format=O.MXFP4)
    x, xr = dev(x_h), dev(xr_h)
    rc, rs = fq.fp4_quantize(xr, cfg, None)
    gb, gs = fq.guide_pack(rc, rs, cfg, rows, cols)
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(-23131)   # 0xA5A5
    fq.fp4_fake_quantize(x, cfg, None, gb, gs, out=out)          # as bench.py times it
    torch.cuda.synchronize()
    idx = sample_rows(rows, 48, seed=50)
    for r in idx:
        orc, ors = O.quantize(oc, O.RTN, xr_h[r:r + 1], row0=r)
        ogb, ogs = O.guide_pack(oc, orc, ors, 1, cols)
        ogc, ogsc = O.quantize(oc, O.GUIDED, x_h[r:r + 1], row0=r, guide_bits=ogb, guide_scales=ogs)
        want = O.dequantize(oc, ogc, ogsc, 1.0, 1, cols, out_bf16=True)
        assert (out[r].view(torch.int16).cpu().numpy() == want.view(np.int16)).all(), r
    say(f"C2 guided fake quantization: {len(idx)} rows bit-exact ({time.time() - t0:.1f} s)")


def test_c1_sixteen_tensors_grouped(fq):
    rows, cols = W.c1_shape()
    t0 = time.time()
    G = 16
    cfg, oc = fq.Fp4Config(), O.Cfg()
    xh, xrh = W.c1_x(rows, cols), W.c1_rollout(rows, cols)
    x0 = dev(xh)
    xs = [torch.roll(x0, s * 61, 0) for s in range(G)]      # as bench.py rotates its copies
    # rotating rows leaves the maximum alone: one tensor scale, the rollout's, for every copy
    ts = fq.fp4_tensor_scale(dev(xrh), cfg)
    o_ts = O.tensor_scale(oc, xrh)
    assert f32bits(ts.item()) == f32bits(o_ts)
    n = rows * cols
    outs = [(poisoned(n // 2), poisoned(n // 16)) for _ in range(G)]
    fq.fp4_quantize_grouped(xs, cfg, [ts] * G, outs=outs)       # as bench.py times it
    torch.cuda.synchronize()
    for t in range(G):
        c, sc = outs[t]
        for r in sample_rows(rows, 8, seed=60 + t):
            src = (r - 61 * t) % rows
            oc_r, os_r = O.quantize(oc, O.RTN, xh[src:src + 1], o_ts, row0=r)
            assert (rows_of(c, r, cols // 2) == oc_r).all(), ("codes", t, r)
            assert (rows_of(sc, r, cols // 16) == os_r).all(), ("scales", t, r)
    say(f"C1 x 16 grouped: {G} tensors, sampled rows bit-exact ({time.time() - t0:.1f} s)")
