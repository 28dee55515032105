"""Fake quantization (quantize -> dequantize in one pass) equals the oracle's
dequantize(quantize(x)) in bf16, bit for bit, in every mode; the autograd
wrapper passes gradients straight through."""
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


@pytest.mark.parametrize("fmt,grid,rnd,rht", [(0, 0, 0, False), (1, 0, 0, False), (1, 0, 1, False),
                                              (0, 1, 1, True), (0, 0, 1, True), (1, 1, 0, False),
                                              (1, 0, 1, True), (1, 1, 0, True)])
@pytest.mark.parametrize("shape,pad", [((256, 512), 0), ((37, 544), 24), ((1, 64), 0), ((1031, 1056), 8)])
def test_fake_quantize_vs_oracle(fq, fmt, grid, rnd, rht, shape, pad):
    rows, cols = shape
    if cols % (32 if fmt else 16):
        pytest.skip("shape not valid for this block size")
    xh = W.c5_x(rows, cols, seed=rows)
    xh[0, :16] = W.f32_to_bf16_rne(np.zeros(16, np.float32))
    cfg = fq.Fp4Config(format=fmt, grid=grid, rounding=rnd, rht16=rht, rht_seed=7, sr_seed=5)
    oc = O.Cfg(format=fmt, grid=grid, rht16=rht, rht_seed=7, sr_seed=5)
    x = dev(xh, pad)
    ts = fq.fp4_tensor_scale(x, cfg) if fmt == 0 else None
    o_ts = O.tensor_scale(oc, xh) if fmt == 0 else 1.0
    out = torch.zeros((rows, cols + pad), dtype=torch.bfloat16, device="cuda")[:, :cols]
    fq.fp4_fake_quantize(x, cfg, ts, out=out)
    c, s = O.quantize(oc, rnd, xh, o_ts)
    want = O.dequantize(oc, c, s, o_ts, rows, cols, out_bf16=True).reshape(rows, cols)
    got = out.contiguous().view(torch.int16).cpu().numpy()
    assert (got == want.view(np.int16)).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_guided_fake_quantize_vs_oracle(fq, fmt):
    rows, cols = 64, 512
    x_h, xr_h = W.c1_x(rows, cols, seed=4), W.c1_rollout(rows, cols, seed=4)
    cfg = fq.Fp4Config(format=fmt)
    oc = O.Cfg(format=fmt)
    xr = dev(xr_h)
    ts = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    _, rs, gb = fq.fp4_quantize(xr, cfg, ts, emit=True)
    out = fq.fp4_fake_quantize(dev(x_h), cfg, ts, gb, rs)
    o_ts = O.tensor_scale(oc, xr_h) if fmt == 0 else 1.0
    _, o_rs, o_gb = O.quantize(oc, O.RTN, xr_h, o_ts, emit=True)
    gc, gs = O.quantize(oc, O.GUIDED, x_h, o_ts, guide_bits=o_gb, guide_scales=o_rs)
    want = O.dequantize(oc, gc, gs, o_ts, rows, cols, out_bf16=True)
    assert (out.view(torch.int16).cpu().numpy().reshape(-1) == want.view(np.int16)).all()


def test_straight_through_gradient(fq):
    from precision_rl_amd.autograd import fake_quantize_ste
    rows, cols = 32, 256
    x = dev(W.c1_x(rows, cols, seed=1)).clone().requires_grad_(True)
    w = torch.randn(rows, cols, device="cuda").to(torch.bfloat16)
    cfg = fq.Fp4Config()
    y = fake_quantize_ste(x, cfg)
    ref = fq.fp4_fake_quantize(x.detach(), cfg, fq.fp4_tensor_scale(x.detach(), cfg))
    assert torch.equal(y.detach(), ref)
    (y.float() * w.float()).sum().backward()
    assert torch.equal(x.grad, w)


@pytest.mark.parametrize("fmt", [0, 1])
def test_guided_straight_through_vs_oracle(fq, fmt):
    # The guided QAT path through autograd: the forward value is the oracle's guided rounding of x
    # under the rollout's guide (its bits, block scales and, for NVFP4, tensor scale); the backward
    # pass hands the incoming gradient through unchanged.  Guided NVFP4 without the guide's tensor
    # scale is refused.
    from precision_rl_amd.autograd import fake_quantize_ste
    rows, cols = 96, 1024
    x_h, xr_h = W.c1_x(rows, cols, seed=12), W.c1_rollout(rows, cols, seed=12)
    cfg = fq.Fp4Config(format=fmt)
    oc = O.Cfg(format=fmt)
    xr = dev(xr_h)
    ts = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    _, rs, gb = fq.fp4_quantize(xr, cfg, ts, emit=True)
    x = dev(x_h).clone().requires_grad_(True)
    y = fake_quantize_ste(x, cfg, ts, gb, rs)
    o_ts = O.tensor_scale(oc, xr_h) if fmt == 0 else 1.0
    _, o_rs, o_gb = O.quantize(oc, O.RTN, xr_h, o_ts, emit=True)
    gc, gs = O.quantize(oc, O.GUIDED, x_h, o_ts, guide_bits=o_gb, guide_scales=o_rs)
    want = O.dequantize(oc, gc, gs, o_ts, rows, cols, out_bf16=True)
    assert (y.detach().view(torch.int16).cpu().numpy().reshape(-1) == want.view(np.int16)).all()
    g = torch.randn(rows, cols, device="cuda").to(torch.bfloat16)
    y.backward(g)
    assert torch.equal(x.grad, g)
    if fmt == 0:
        with pytest.raises(ValueError):
            fake_quantize_ste(x, cfg, None, gb, rs)
