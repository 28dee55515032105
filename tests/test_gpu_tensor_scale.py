"""The one-launch tensor scale (fp4_tensor_scale_ws) equals the oracle's tensor
scale and the three-launch fp4_tensor_scale bit for bit: small and large
tensors (both launch shapes, one pass of up to 512 workgroups and the
grid-stride form with 1024), every grid size from 1 to 18 workgroups (the
workgroup words gathered in one or several loads per thread) and others up
to the 1024 cap, with and without a one-group last workgroup, ragged tails,
padded rows, the RHT, both grids, all-zero, empty and non-finite inputs.  One
workspace serves every call in turn: each call advances its epoch by one and
tags every workgroup's word with it (and without the RHT, the largest word is
the tensor's largest finite |x|).  A captured graph of calls replays equal to
eager calls."""
import numpy as np
import pytest
import torch

import oracle as O
from precision_rl_amd import workloads as W
from ts_workspace import chunk_max_bits, check_after, epoch, mark, ts_grid

pytestmark = pytest.mark.gpu

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


@pytest.mark.parametrize("rht,grid", [(False, 0), (True, 1), (True, 0)])
@pytest.mark.parametrize("shape,pad", [((3, 16), 0), ((5, 48), 8), ((129, 96), 0), ((1, 16 * 1027), 0),
                                       ((4096, 2048), 0), ((1000, 2080), 16), ((4096, 8192), 0)])
def test_one_launch_tensor_scale_vs_oracle(fq, ws, rht, grid, shape, pad):
    rows, cols = shape
    xh = W.c5_x(rows, cols, seed=rows + cols)
    cfg = fq.Fp4Config(grid=grid, rht16=rht, rht_seed=7)
    oc = O.Cfg(grid=grid, rht16=rht, rht_seed=7)
    x = dev(xh, pad)
    e0 = epoch(ws)
    got = fq.fp4_tensor_scale_ws(x, cfg, ws)
    want = np.float32(O.tensor_scale(oc, xh)).view(np.uint32)
    assert bits(got) == want
    check_after(ws, e0, ts_grid(rows * cols // 16),
                amax_bits=None if rht else int(chunk_max_bits(xh, rows * cols).max()))
    three = fq.fp4_tensor_scale(x, cfg)
    assert bits(three) == want


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
    e0 = epoch(ws)
    got = fq.fp4_tensor_scale_ws(dev(flat), cfg, ws)
    assert bits(got) == np.float32(O.tensor_scale(O.Cfg(), flat)).view(np.uint32)
    # up to 1024 workgroups, workgroup b takes row b (1024 groups)
    check_after(ws, e0, ts_grid(n // 16), wg_max_bits=chunk_max_bits(flat, cols) if k <= 1024 else None,
                amax_bits=int(chunk_max_bits(flat, n).max()))


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
    e0 = epoch(ws)
    got = fq.fp4_tensor_scale_ws(dev(xh), cfg, ws)
    assert bits(got) == np.float32(O.tensor_scale(oc, xh)).view(np.uint32)
    check_after(ws, e0, ts_grid(300 * 512 // 16), amax_bits=int(chunk_max_bits(xh, xh.size).max()))
    # a workspace zero-filled again is a valid start
    ws.zero_()
    got = fq.fp4_tensor_scale_ws(dev(xh), cfg, ws)
    assert bits(got) == np.float32(O.tensor_scale(oc, xh)).view(np.uint32)
    check_after(ws, 0, ts_grid(300 * 512 // 16))


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
        e0 = epoch(ws)
        fq.fp4_tensor_scale_ws(xs[rep], cfg, ws, out=outs[rep])
        assert bits(outs[rep]) == want[rep]
        check_after(ws, e0, ts_grid(2048 * 2048 // 16))


def test_wait_gives_up_with_nan_and_workspace_recovers(fq, ws):
    # a wait limit of 0 makes workgroup 0's gather give up at once: s_t is NaN, the epoch still
    # advances with the launch's give-up mark beside it (workgroups of that launch that start later
    # store nothing), and the next call with the default limit is exact again and clears the mark
    L = fq.lib()
    cfg = fq.Fp4Config()
    # 512 workgroups; every chunk maximum of this tensor is far above any value of the next one, so
    # a word left over from this launch and taken by the next call's gather would change its s_t
    xf = np.random.default_rng(77).standard_normal((512, 16384)).astype(np.float32) * 4096.0
    x = dev(W.f32_to_bf16_rne(xf))
    e0 = epoch(ws)
    prev = L.fp4_set_wait_limit(0)
    try:
        got = fq.fp4_tensor_scale_ws(x, cfg, ws)
        torch.cuda.synchronize()
    finally:
        L.fp4_set_wait_limit(prev)
    assert np.isnan(got.cpu().numpy()[0])
    assert epoch(ws) == e0 + 1 and mark(ws) != 0
    e1 = epoch(ws)
    xh2 = W.c1_x(512, 16384, seed=79)
    want2 = np.float32(O.tensor_scale(O.Cfg(), xh2)).view(np.uint32)
    assert bits(fq.fp4_tensor_scale_ws(dev(xh2), cfg, ws)) == want2
    check_after(ws, e1, ts_grid(512 * 16384 // 16), amax_bits=int(chunk_max_bits(xh2, xh2.size).max()))
