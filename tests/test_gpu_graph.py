"""HIP-graph capture and concurrent streams.

The library enqueues kernels only (no memsets, allocations or synchronizations),
so its calls can be captured in a HIP graph.  A graph of tensor scale, RTN
quantize with emission, guide_pack, guided quantize and dequantize is replayed
several times, with eager work of the same calls in between, and every replay's
outputs must equal the eager results bit for bit.  Two streams running
different configurations at once must give the results of running them one
after the other (the library keeps no state between calls).
"""
import numpy as np
import pytest
import torch

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


def u8(n):
    return torch.empty(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("fmt", [0, 1])
def test_graph_replays_equal_eager(fq, fmt):
    rows, cols = 300, 1024
    n = rows * cols
    B = 32 if fmt else 16
    x, xr = dev(W.c1_x(rows, cols, seed=5)), dev(W.c1_rollout(rows, cols, seed=5))
    cfg = fq.Fp4Config(format=fmt)
    ts = torch.empty(1, dtype=torch.float32, device="cuda") if fmt == 0 else None
    rc, rs, rb = u8(n // 2), u8(n // B), u8(n // 8)
    gb, gs = u8(n // 8), u8(n // B)
    gc, gsc = u8(n // 2), u8(n // B)
    dq = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")

    def pipeline():
        if fmt == 0:
            fq.fp4_tensor_scale(xr, cfg, out=ts)
        fq.fp4_quantize(xr, cfg, ts, emit=True, codes=rc, scales=rs, bits=rb)
        fq.guide_pack(rc, rs, cfg, rows, cols, bits=gb, gscales=gs)
        fq.fp4_quantize_guided(x, cfg, gb, gs, ts, codes=gc, scales=gsc)
        fq.fp4_dequantize(gc, gsc, cfg, rows, cols, ts, out=dq)

    outs = [rc, rs, rb, gb, gs, gc, gsc, dq] + ([ts] if fmt == 0 else [])
    pipeline()
    torch.cuda.synchronize()
    want = [t.clone() for t in outs]
    # capture on a side stream (torch's graph capture), then clobber the outputs eagerly
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pipeline()   # warm the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        pipeline()
    for rep in range(3):
        for t in outs:
            t.zero_() if t.dtype != torch.float32 else t.fill_(-1.0)
        # eager work of the same calls on other inputs between the replays
        other = dev(W.c1_x(rows, cols, seed=100 + rep))
        fq.fp4_quantize(other, cfg, fq.fp4_tensor_scale(other, cfg) if fmt == 0 else None)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, want)):
            assert torch.equal(a, b), (rep, i)


def test_two_streams_equal_serial(fq):
    rows, cols = 512, 2048
    xa, xb = dev(W.c2_pair(rows, cols, seed=3)[0]), dev(W.c5_x(rows, cols, seed=4))
    ca = fq.Fp4Config(format=fq.MXFP4, rounding=fq.SR, sr_seed=11)
    cb = fq.Fp4Config(grid=fq.UNIFORM, rounding=fq.SR, rht16=True, rht_seed=7, sr_seed=5)
    tsb = fq.fp4_tensor_scale(xb, cb)
    want_a = fq.fp4_quantize(xa, ca)
    want_b = fq.fp4_quantize(xb, cb, tsb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    got_a, got_b = [], []
    for _ in range(8):
        with torch.cuda.stream(s1):
            got_a.append(fq.fp4_quantize(xa, ca))
        with torch.cuda.stream(s2):
            got_b.append(fq.fp4_quantize(xb, cb, tsb))
    torch.cuda.synchronize()
    for a in got_a:
        assert torch.equal(a[0], want_a[0]) and torch.equal(a[1], want_a[1])
    for b in got_b:
        assert torch.equal(b[0], want_b[0]) and torch.equal(b[1], want_b[1])
