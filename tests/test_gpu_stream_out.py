"""fp4_cfg.stream_out = 1 (non-temporal stores for outputs not read again soon)
changes no output: every quantize path gives the same codes, scales, guide bits
and fake-quantized values bit for bit as with stream_out = 0, and the same as
the oracle on a sampled case.  Covered: RTN with emission, SR and guided in both
formats, the uniform grid with the RHT and SR, both slot counts (2048 x 4096
NVFP4 SR takes four), grouped RTN with emission and grouped guided, guided fake
quantization, and the tensor scale + quantize in one launch and in two.
Outputs start as 0xA5 bytes (the conftest fixture)."""
import dataclasses

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


def dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def same(a, b):
    torch.cuda.synchronize()
    assert len(a) == len(b)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def streamed(cfg):
    return dataclasses.replace(cfg, stream_out=True)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rows", [300, 4096])
def test_quantize_modes(fq, fmt, rows):
    cols = 2048
    xh = W.c1_x(rows, cols, seed=rows + fmt)
    x = dev(xh)
    cfg = fq.Fp4Config(format=fmt)
    ts = fq.fp4_tensor_scale(x, cfg) if fmt == 0 else None
    rtn = fq.fp4_quantize(x, cfg, ts, emit=True)
    same(rtn, fq.fp4_quantize(x, streamed(cfg), ts, emit=True))
    sr = fq.Fp4Config(format=fmt, rounding=fq.SR, sr_seed=11, sr_offset=3)
    same(fq.fp4_quantize(x, sr, ts), fq.fp4_quantize(x, streamed(sr), ts))
    g = fq.fp4_quantize_guided(x, cfg, rtn[2], rtn[1], ts)
    same(g, fq.fp4_quantize_guided(x, streamed(cfg), rtn[2], rtn[1], ts))
    # the streamed RTN against the oracle
    oc = O.Cfg(format=fmt)
    ots = O.tensor_scale(oc, xh) if fmt == 0 else 1.0
    wc, ws, wb = O.quantize(oc, O.RTN, xh, ots, emit=True)
    c, s, b = fq.fp4_quantize(x, streamed(cfg), ts, emit=True)
    torch.cuda.synchronize()
    assert (c.cpu().numpy() == wc).all() and (s.cpu().numpy() == ws).all() and (b.cpu().numpy() == wb).all()


def test_uniform_rht_sr(fq):
    x = dev(W.c5_x(512, 2048, seed=8))
    cfg = fq.Fp4Config(grid=fq.UNIFORM, rounding=fq.SR, rht16=True, rht_seed=3, sr_seed=9)
    ts = fq.fp4_tensor_scale(x, cfg)
    same(fq.fp4_quantize(x, cfg, ts), fq.fp4_quantize(x, streamed(cfg), ts))


def test_grouped_and_fake(fq):
    xs = [dev(W.c1_x(r, c, seed=r)) for r, c in ((256, 1536), (64, 4096), (129, 512))]
    cfg = fq.Fp4Config()
    tss = [fq.fp4_tensor_scale(x, cfg) for x in xs]
    a = fq.fp4_quantize_grouped(xs, cfg, tss, emit=True)
    same([t for o in a for t in o], [t for o in fq.fp4_quantize_grouped(xs, streamed(cfg), tss, emit=True) for t in o])
    guides = [(o[2], o[1]) for o in a]
    g0 = fq.fp4_quantize_grouped(xs, cfg, tss, guides=guides)
    g1 = fq.fp4_quantize_grouped(xs, streamed(cfg), tss, guides=guides)
    same([t for o in g0 for t in o], [t for o in g1 for t in o])
    x = xs[0]
    f0 = fq.fp4_fake_quantize(x, cfg, tss[0], a[0][2], a[0][1])
    f1 = fq.fp4_fake_quantize(x, streamed(cfg), tss[0], a[0][2], a[0][1])
    same([f0], [f1])


def test_quantize_with_tensor_scale(fq):
    ws = fq.tensor_scale_workspace()
    cfg = fq.Fp4Config()
    for rows, cols, launches in ((1024, 2048, 1), (8192, 4096, 2)):
        x = dev(W.c1_x(rows, cols, seed=rows))
        a = fq.fp4_quantize_with_tensor_scale(x, cfg, ws, emit=True)
        assert fq.last_launches == launches
        b = fq.fp4_quantize_with_tensor_scale(x, streamed(cfg), ws, emit=True)
        assert fq.last_launches == launches
        same(a, b)
