"""Grouped quantization (several tensors, one launch) equals the oracle on each
tensor, in every mode, with mixed shapes, padded rows and a ragged tail."""
import numpy as np
import pytest
import torch

import oracle as O
from precision_rl_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from precision_rl_amd import fp4q
    fp4q.lib()
    return fp4q


def dev(u16, pad=0):
    rows, cols = u16.shape
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
    if pad:
        buf = torch.full((rows, cols + pad), float("nan"), dtype=torch.bfloat16)
        buf[:, :cols] = t
        return buf.cuda()[:, :cols]
    return t.cuda()


SHAPES = [(37, 544), (256, 512), (1, 64), (129, 96), (64, 1536), (8, 4096), (3, 32)]


@pytest.mark.parametrize("fmt,grid,rnd,rht", [(0, 0, 0, False), (1, 0, 0, False), (1, 0, 1, False),
                                              (0, 1, 1, True), (0, 0, 1, False)])
def test_grouped_rtn_sr_with_emission(fq, fmt, grid, rnd, rht):
    B = 32 if fmt else 16
    shapes = [(r, c) for r, c in SHAPES if c % B == 0]
    cfg = fq.Fp4Config(format=fmt, grid=grid, rounding=rnd, rht16=rht, rht_seed=7, sr_seed=99, sr_offset=5)
    oc = O.Cfg(format=fmt, grid=grid, rht16=rht, rht_seed=7, sr_seed=99, sr_offset=5)
    hs = [W.c5_x(r, c, seed=i) for i, (r, c) in enumerate(shapes)]
    xs = [dev(h, pad=8 * (i % 2)) for i, h in enumerate(hs)]
    tss = [fq.fp4_tensor_scale(x, cfg) for x in xs] if fmt == 0 else None
    outs = fq.fp4_quantize_grouped(xs, cfg, tss, emit=True)
    torch.cuda.synchronize()
    for i, h in enumerate(hs):
        ts = O.tensor_scale(oc, h) if fmt == 0 else 1.0
        c, s, b = O.quantize(oc, rnd, h, ts, emit=True)
        assert (outs[i][0].cpu().numpy() == c).all(), i
        assert (outs[i][1].cpu().numpy() == s).all(), i
        assert (outs[i][2].cpu().numpy() == b).all(), i


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_guided(fq, fmt):
    B = 32 if fmt else 16
    shapes = [(r, c) for r, c in SHAPES if c % B == 0]
    cfg = fq.Fp4Config(format=fmt)
    oc = O.Cfg(format=fmt)
    xh = [W.c1_x(r, c, seed=i) for i, (r, c) in enumerate(shapes)]
    xrh = [W.c1_rollout(r, c, seed=i) for i, (r, c) in enumerate(shapes)]
    xs, xrs = [dev(h) for h in xh], [dev(h, pad=16) for h in xrh]
    tss = [fq.fp4_tensor_scale(x, cfg) for x in xrs] if fmt == 0 else None
    roll = fq.fp4_quantize_grouped(xrs, cfg, tss, emit=True)
    guides = [(o[2], o[1]) for o in roll]
    got = fq.fp4_quantize_grouped(xs, cfg, tss, guides=guides)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        ts = O.tensor_scale(oc, xrh[i]) if fmt == 0 else 1.0
        rc, rs, rb = O.quantize(oc, O.RTN, xrh[i], ts, emit=True)
        gc, gs = O.quantize(oc, O.GUIDED, xh[i], ts, guide_bits=rb, guide_scales=rs)
        assert (got[i][0].cpu().numpy() == gc).all(), i
        assert (got[i][1].cpu().numpy() == gs).all(), i


def test_grouped_sixteen_tensors_equal_single_calls(fq):
    cfg = fq.Fp4Config(format=1, rounding=1, sr_seed=3)
    hs = [W.c2_pair(16 + 7 * i, 256, seed=i)[0] for i in range(16)]
    xs = [dev(h) for h in hs]
    grouped = fq.fp4_quantize_grouped(xs, cfg)
    for x, g in zip(xs, grouped):
        c, s = fq.fp4_quantize(x, cfg)
        assert torch.equal(c, g[0]) and torch.equal(s, g[1])


@pytest.mark.parametrize("fmt", [0, 1])
def test_grouped_guide_pack(fq, fmt):
    # codes and scales from the oracle's quantization of mixed shapes (odd NVFP4 group counts included);
    # one grouped launch equals the oracle's guide_pack on each tensor, bit for bit
    B = 32 if fmt else 16
    shapes = [(r, c) for r, c in SHAPES + [(3, 48), (5, 16)] if c % B == 0]
    oc = O.Cfg(format=fmt)
    cfg = fq.Fp4Config(format=fmt)
    host, tensors = [], []
    for i, (r, c) in enumerate(shapes):
        h = W.c1_x(r, c, seed=40 + i)
        ts = O.tensor_scale(oc, h) if fmt == 0 else 1.0
        codes, scales = O.quantize(oc, O.RTN, h, ts)
        host.append((codes, scales, r, c))
        tensors.append((torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), r, c))
    outs = fq.guide_pack_grouped(tensors, cfg)
    torch.cuda.synchronize()
    for i, (codes, scales, r, c) in enumerate(host):
        bits, gs = O.guide_pack(oc, codes, scales, r, c)
        assert (outs[i][0].cpu().numpy() == bits).all(), i
        assert (outs[i][1].cpu().numpy() == gs).all(), i
