"""fp4_quantize_with_tensor_scale: the NVFP4 tensor scale and the block
quantization of one tensor together.  Where the launch is one kernel (no RHT,
grid within what the device holds at once) and where it is two (RHT, or a grid
too large), s_t must equal the oracle's tensor scale bit for bit and the codes,
scales and guide bits the oracle's quantization with that s_t.  After each call
the workspace's epoch has advanced by one, every workgroup's word carries it
(in the one-launch form, with exactly its own chunk's largest finite |x|) and
so do the published copies of s_t.  Covered: every grid size from
1 to 9 workgroups (a workgroup quantizes 512 groups of 16) and others up to the
one-launch limit and past it, ragged tails, padded rows, both grids, RTN with and
without emission and SR, all-zero, empty and non-finite inputs, replays of a
captured HIP graph against eager calls, and a workspace zero-filled between calls
(a valid state at any time).  Outputs start as 0xA5 bytes (the
conftest fixture)."""
import numpy as np
import pytest
import torch

import oracle as O
from precision_rl_amd import workloads as W
from ts_workspace import chunk_max_bits, check_after, epoch, fused_grid, mark, ts_grid

pytestmark = pytest.mark.gpu

CHUNK = 512 * 16          # elements one workgroup of the one-launch form quantizes


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


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits32(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def check(fq, ws, xh, cfg, emit, pad=0, launches=None):
    oc = O.Cfg(grid=cfg.grid, rht16=cfg.rht16, rht_seed=cfg.rht_seed, sr_seed=cfg.sr_seed, sr_offset=cfg.sr_offset)
    mode = O.SR if cfg.rounding == 1 else O.RTN
    e0 = epoch(ws)
    out = fq.fp4_quantize_with_tensor_scale(dev(xh, pad), cfg, ws, emit=emit)
    got_launches = fq.last_launches
    ts = O.tensor_scale(oc, xh)
    assert bits32(host(out[0]))[0] == bits32([ts])[0], (host(out[0]), ts)
    want = O.quantize(oc, mode, xh, ts, emit=emit)
    assert (host(out[2]) == want[1]).all(), "scales"
    assert (host(out[1]) == want[0]).all(), "codes"
    if emit:
        assert (host(out[3]) == want[2]).all(), "guide bits"
    if launches is not None:
        assert got_launches == launches
    ng = xh.size // 16
    if got_launches == 1:
        check_after(ws, e0, fused_grid(ng), ts_bits=bits32([ts])[0], wg_max_bits=chunk_max_bits(xh, CHUNK))
    else:
        check_after(ws, e0, ts_grid(ng), amax_bits=None if cfg.rht16 else int(chunk_max_bits(xh, xh.size).max()))
    return got_launches


@pytest.mark.parametrize("k", list(range(1, 10)) + [16, 17, 255, 1024])
def test_grid_sizes_one_launch(fq, ws, k):
    # k workgroups; the largest magnitude sits in the last one
    xh = W.c1_x(k, CHUNK, seed=k).copy()
    xh[-1, 5] = W.f32_to_bf16_rne(np.array([[-977.0]], dtype=np.float32))[0, 0]
    check(fq, ws, xh, fq.Fp4Config(), emit=True, launches=1)


@pytest.mark.parametrize("rows", [1, 3, 255])
def test_one_group_last_workgroup(fq, ws, rows):
    # the last workgroup holds a single group: (rows - 1) full chunks plus 16 elements
    xh = W.c1_x(1, (rows - 1) * CHUNK + 16, seed=rows)
    check(fq, ws, xh, fq.Fp4Config(), emit=False, launches=1)


@pytest.mark.parametrize("grid,rounding,emit", [(0, 0, False), (0, 0, True), (0, 1, False), (1, 0, True),
                                                 (1, 1, False)])
@pytest.mark.parametrize("shape,pad", [((1, 16), 0), ((3, 48), 8), ((129, 96), 0), ((37, 544), 24),
                                       ((4096, 2048), 0), ((1000, 2080), 16)])
def test_vs_oracle(fq, ws, grid, rounding, emit, shape, pad):
    rows, cols = shape
    xh = W.c1_x(rows, cols, seed=rows * 7 + cols)
    cfg = fq.Fp4Config(grid=grid, rounding=rounding, sr_seed=0x1234567, sr_offset=5)
    check(fq, ws, xh, cfg, emit, pad=pad, launches=1)


def test_full_size_activation(fq, ws):
    # the NVFP4 activation workload, 4096 x 2048 (1024 workgroups), with its rollout copy
    rows, cols = 4096, 2048
    for xh in (W.c1_x(rows, cols, seed=0), W.c1_rollout(rows, cols, seed=0)):
        check(fq, ws, xh, fq.Fp4Config(), emit=True, launches=1)


def test_two_launch_forms(fq, ws):
    # with the RHT, and for a grid past what the device holds at once (8192 x 4096: 4096 workgroups)
    xh = W.c5_x(96, 512, seed=4)
    check(fq, ws, xh, fq.Fp4Config(rht16=True, rht_seed=7), emit=True, launches=2)
    xh = W.c1_x(8192, 4096, seed=9)
    check(fq, ws, xh, fq.Fp4Config(), emit=False, launches=2)


def test_special_inputs(fq, ws):
    cfg = fq.Fp4Config()
    z = np.zeros((64, 256), dtype=np.uint16)
    check(fq, ws, z, cfg, emit=True, launches=1)
    e0 = epoch(ws)
    ts, codes, scales = fq.fp4_quantize_with_tensor_scale(torch.empty((0, 64), dtype=torch.bfloat16,
                                                                      device="cuda"), cfg, ws)
    assert bits32(host(ts))[0] == bits32([1.0])[0] and codes.numel() == 0
    check_after(ws, e0, 1, amax_bits=0)            # the one-launch tensor scale with one workgroup
    # non-finite values are left out of s_t; their blocks get the NaN scale code
    xf = np.random.default_rng(3).standard_normal((300, 512)).astype(np.float32)
    xf[7, 9], xf[100, 0], xf[299, 511] = np.inf, -np.inf, np.nan
    check(fq, ws, W.f32_to_bf16_rne(xf), cfg, emit=True, launches=1)


def test_zero_filled_workspace_between_calls(fq, ws):
    # zero-filling resets the epoch (and every word); the next calls must still tag, publish and read
    # the right words
    cfg = fq.Fp4Config()
    for k in range(5):
        if k in (1, 3):
            ws.zero_()
        check(fq, ws, W.c1_x(300, 1024, seed=40 + k), cfg, emit=False, launches=1)


def test_graph_replays(fq, ws):
    cfg = fq.Fp4Config()
    xs = [dev(W.c1_x(2048, 2048, seed=s)) for s in range(3)]
    outs = [fq.fp4_quantize_with_tensor_scale(x, cfg, ws, emit=True) for x in xs]   # eager, allocates
    want = [[host(t).copy() for t in o] for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for x, o in zip(xs, outs):
                fq.fp4_quantize_with_tensor_scale(x, cfg, ws, emit=True, ts=o[0], codes=o[1], scales=o[2],
                                                  bits=o[3])
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for o in outs:
            for t in o:
                t.view(torch.uint8).fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            for t, wt in zip(o, w):
                assert (host(t) == wt).all(), rep
        # eager work between the replays
        fq.fp4_quantize_with_tensor_scale(xs[rep], cfg, ws, emit=True)
        torch.cuda.synchronize()


def test_waits_give_up_with_nan_and_workspace_recovers(fq, ws):
    # a wait limit of 0: workgroup 0 publishes s_t = NaN at once and every other workgroup stops
    # waiting at once, so the launch ends with s_t NaN; the next call with the default limit is exact
    L = fq.lib()
    cfg = fq.Fp4Config()
    # 256 workgroups, one launch; every chunk maximum of this tensor is far above any value of the
    # next one, so a word left over from this launch and taken by the next call's gather would show
    xf = np.random.default_rng(78).standard_normal((256, CHUNK)).astype(np.float32) * 4096.0
    e0 = epoch(ws)
    prev = L.fp4_set_wait_limit(0)
    try:
        out = fq.fp4_quantize_with_tensor_scale(dev(W.f32_to_bf16_rne(xf)), cfg, ws, emit=True)
        torch.cuda.synchronize()
    finally:
        L.fp4_set_wait_limit(prev)
    assert fq.last_launches == 1
    assert np.isnan(host(out[0])[0])
    assert epoch(ws) == e0 + 1 and mark(ws) != 0
    check(fq, ws, W.c1_x(256, CHUNK, seed=79), cfg, emit=True, launches=1)
