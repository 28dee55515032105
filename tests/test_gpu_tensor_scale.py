"""The one-launch tensor scale (fp4_tensor_scale_ws) equals the oracle's tensor
scale and the three-launch fp4_tensor_scale bit for bit: small and large
tensors (both launch shapes, one pass of up to 512 workgroups and the
grid-stride form with 1024), every grid size from 1 to 18 workgroups (the
eight reduction slots with zero to three arrivals each) and others up to the
1024 cap, with and without a one-group last workgroup, ragged tails, padded
rows, the RHT, both grids,
all-zero, empty and non-finite inputs.  One workspace serves every call in
turn: each call leaves its maxima and arrival counters at 0.  A captured graph of calls
replays equal to eager calls."""
import numpy as np
import pytest
import torch

import oracle as O
from precision_rl_amd import workloads as W

pytestmark = pytest.mark.gpu

# word offsets of the shared words in the workspace: 8 slot maxima, 8 slot counters, top maximum, top counter
SHARED_WORDS = [64 * k for k in range(18)]


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from precision_rl_amd import fp4q
    fp4q.lib()
    return fp4q


@pytest.fixture(scope="module")
def ws(fq):
    return fq.tensor_scale_workspace()


def dev(u16, pad=0):
    rows, cols = u16.shape
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
    if pad:
        buf = torch.full((rows, cols + pad), float("nan"), dtype=torch.bfloat16)
        buf[:, :cols] = t
        return buf.cuda()[:, :cols]
    return t.cuda()


def bits(t):
    torch.cuda.synchronize()
    return np.float32(t.cpu().numpy()[0]).view(np.uint32)


def counters_zero(ws):
    w = ws.view(torch.int32).cpu().numpy()
    return all(int(w[i]) == 0 for i in SHARED_WORDS)


@pytest.mark.parametrize("rht,grid", [(False, 0), (True, 1), (True, 0)])
@pytest.mark.parametrize("shape,pad", [((3, 16), 0), ((5, 48), 8), ((129, 96), 0), ((1, 16 * 1027), 0),
                                       ((4096, 2048), 0), ((1000, 2080), 16), ((4096, 8192), 0)])
def test_one_launch_tensor_scale_vs_oracle(fq, ws, rht, grid, shape, pad):
    rows, cols = shape
    xh = W.c5_x(rows, cols, seed=rows + cols)
    cfg = fq.Fp4Config(grid=grid, rht16=rht, rht_seed=7)
    oc = O.Cfg(grid=grid, rht16=rht, rht_seed=7)
    x = dev(xh, pad)
    got = fq.fp4_tensor_scale_ws(x, cfg, ws)
    three = fq.fp4_tensor_scale(x, cfg)
    want = np.float32(O.tensor_scale(oc, xh)).view(np.uint32)
    assert bits(got) == want
    assert bits(three) == want
    assert counters_zero(ws)


@pytest.mark.parametrize("k", list(range(1, 19)) + [63, 64, 65, 1023, 1024, 1100])
@pytest.mark.parametrize("tail", [False, True])
def test_one_launch_tensor_scale_grid_sizes(fq, ws, k, tail):
    # a workgroup covers 1024 groups of 16 (16384 elements), so k rows of 16384 make k workgroups
    # (at most 1024): slot b mod 8 of the reduction gets ceil((k - b) / 8) arrivals, and slots past
    # k - 1 none.  With the tail the last row is one group long, so the last workgroup holds a
    # single group.  The largest value sits in the last workgroup.
    cols = 16384
    xh = W.c1_x(k, cols, seed=k)
    if tail:
        xh = xh.copy()
        xh[-1, 16:] = 0
        xh[-1, 3] = W.f32_to_bf16_rne(np.array([[-977.0]], dtype=np.float32))[0, 0]
    n = (k - 1) * cols + (16 if tail else cols)
    flat = np.ascontiguousarray(xh).reshape(-1)[:n].reshape(1, n)
    cfg = fq.Fp4Config()
    got = fq.fp4_tensor_scale_ws(dev(flat), cfg, ws)
    assert bits(got) == np.float32(O.tensor_scale(O.Cfg(), flat)).view(np.uint32)
    assert counters_zero(ws)


def test_one_launch_tensor_scale_special_inputs(fq, ws):
    cfg = fq.Fp4Config()
    oc = O.Cfg()
    z = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    assert bits(fq.fp4_tensor_scale_ws(z, cfg, ws)) == np.float32(1.0).view(np.uint32)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert bits(fq.fp4_tensor_scale_ws(e, cfg, ws)) == np.float32(1.0).view(np.uint32)
    # non-finite values are left out of the maximum
    xf = np.random.default_rng(3).standard_normal((300, 512)).astype(np.float32)
    xf[7, 9], xf[100, 0], xf[299, 511] = np.inf, -np.inf, np.nan
    xh = W.f32_to_bf16_rne(xf)
    got = fq.fp4_tensor_scale_ws(dev(xh), cfg, ws)
    assert bits(got) == np.float32(O.tensor_scale(oc, xh)).view(np.uint32)
    assert counters_zero(ws)


def test_one_launch_tensor_scale_in_a_graph(fq, ws):
    cfg = fq.Fp4Config(rht16=True, rht_seed=3)
    xs = [dev(W.c1_x(2048, 2048, seed=s)) for s in range(3)]
    outs = [torch.empty(1, dtype=torch.float32, device="cuda") for _ in xs]
    want = [bits(fq.fp4_tensor_scale(x, cfg)) for x in xs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fq.fp4_tensor_scale_ws(xs[0], cfg, ws, out=outs[0])     # warm up outside the capture
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for x, o in zip(xs, outs):
                fq.fp4_tensor_scale_ws(x, cfg, ws, out=o)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o in outs:
            o.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert [bits(o) for o in outs] == want, rep
        # eager work between the replays
        fq.fp4_tensor_scale_ws(xs[rep], cfg, ws, out=outs[rep])
        assert bits(outs[rep]) == want[rep]
    assert counters_zero(ws)
