"""GPU parity at the full workload sizes, in the launch configuration bench.py
times.  Every tensor is quantized whole on the GPU; the oracle recomputes
sampled rows (first, last and random rows; its per-row computation uses the
tensor's global element index, so stochastic rounding is checked at its true
counter values) and the comparison is bit for bit.  Tensor scales are
compared exactly against the oracle's whole-tensor reduction.  Whole-tensor
properties: the own-RTN guide reproduces RTN, fused emission equals
guide_pack, and the guidance cache is 1/6 of the full codes for the deep half.
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
    print("[fullsize]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from precision_rl_amd import fp4q
    fq_lib = fp4q.lib()
    return fp4q


def dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def sample_rows(rows, k=48, seed=0):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(k, rows - k), size=k, replace=False) if rows > 3 * k else np.array([], int)
    return sorted(set(range(min(k, rows))) | set(range(max(0, rows - k), rows)) | set(int(r) for r in mid))


def check_rows(fq, cfg, mode, xh, codes, scales, ts, rows_idx, gb=None, gs=None, bits=None, tag=""):
    """Oracle on each sampled row (whole-tensor index via row0) vs the GPU output rows."""
    cols = xh.shape[1]
    B = 32 if cfg.format else 16
    oc = O.Cfg(format=cfg.format, grid=cfg.grid, rht16=cfg.rht16, rht_seed=cfg.rht_seed,
               sr_seed=cfg.sr_seed, sr_offset=cfg.sr_offset)
    c = codes.cpu().numpy().reshape(-1, cols // 2)
    s = scales.cpu().numpy().reshape(-1, cols // B)
    b = bits.cpu().numpy().reshape(-1, cols // 8) if bits is not None else None
    gbr = gb.reshape(-1, cols // 8) if gb is not None else None
    gsr = gs.reshape(-1, cols // B) if gs is not None else None
    for r in rows_idx:
        kw = {}
        if mode == O.GUIDED:
            kw = dict(guide_bits=gbr[r], guide_scales=gsr[r])
        out = O.quantize(oc, mode, xh[r:r + 1], ts, row0=r, emit=b is not None, **kw)
        assert (out[1] == s[r]).all(), (tag, "scales", r)
        assert (out[0] == c[r]).all(), (tag, "codes", r)
        if b is not None:
            assert (out[2] == b[r]).all(), (tag, "bits", r)


def f32bits(x):
    return np.float32(x).view(np.uint32)


def test_c1_nvfp4_activation_4096x2048(fq):
    rows, cols = W.c1_shape()
    t = time.time()
    x_h, xr_h = W.c1_x(rows, cols), W.c1_rollout(rows, cols)
    cfg = fq.Fp4Config()
    oc = O.Cfg()
    x, xr = dev(x_h), dev(xr_h)
    ts = fq.fp4_tensor_scale(xr, cfg)
    o_ts = O.tensor_scale(oc, xr_h)
    assert f32bits(ts.item()) == f32bits(o_ts)
    rc, rs, gb = fq.fp4_quantize(xr, cfg, ts, emit=True)
    # the whole tensor is small enough for the oracle
    o_rc, o_rs, o_gb = O.quantize(oc, O.RTN, xr_h, o_ts, emit=True)
    assert (rc.cpu().numpy() == o_rc).all() and (rs.cpu().numpy() == o_rs).all()
    assert (gb.cpu().numpy() == o_gb).all()
    gc, gs = fq.fp4_quantize_guided(x, cfg, gb, rs, ts)
    o_gc, _ = O.quantize(oc, O.GUIDED, x_h, o_ts, guide_bits=o_gb, guide_scales=o_rs)
    assert (gc.cpu().numpy() == o_gc).all()
    say(f"C1 full tensor bit-exact ({time.time() - t:.1f} s)")


@pytest.mark.parametrize("mode", ["rtn", "sr", "guided"])
def test_c2_mxfp4_moe_activations_16384x4096(fq, mode):
    rows, cols = W.c2_shape()
    t = time.time()
    x_h, xr_h = W.c2_pair(rows, cols, seed=1)
    x = dev(x_h)
    idx = sample_rows(rows)
    if mode == "rtn":
        cfg = fq.Fp4Config(format=fq.MXFP4)
        c, s, b = fq.fp4_quantize(x, cfg, None, emit=True)
        check_rows(fq, cfg, O.RTN, x_h, c, s, 1.0, idx, bits=b, tag="c2 rtn")
        # own-RTN guide reproduces RTN on the whole tensor
        gc, _ = fq.fp4_quantize_guided(x, cfg, b, s, None)
        assert torch.equal(gc, c)
    elif mode == "sr":
        cfg = fq.Fp4Config(format=fq.MXFP4, rounding=fq.SR, sr_seed=W.C2_SR_SEED)
        c, s = fq.fp4_quantize(x, cfg, None)
        check_rows(fq, cfg, O.SR, x_h, c, s, 1.0, idx, tag="c2 sr")
        c2, _ = fq.fp4_quantize(x, cfg, None)
        assert torch.equal(c, c2)  # deterministic for a fixed key and offset
    else:
        cfg = fq.Fp4Config(format=fq.MXFP4)
        xr = dev(xr_h)
        rc, rs = fq.fp4_quantize(xr, cfg, None)
        gb, gs = fq.guide_pack(rc, rs, cfg, rows, cols)
        gc, gsc = fq.fp4_quantize_guided(x, cfg, gb, gs, None)
        assert torch.equal(gsc, rs)
        check_rows(fq, cfg, O.GUIDED, x_h, gc, gsc, 1.0, idx, gb=gb.cpu().numpy(), gs=gs.cpu().numpy(),
                   tag="c2 guided")
    say(f"C2 {mode}: {len(idx)} rows bit-exact ({time.time() - t:.1f} s)")


def test_c3_kv_cache_131072_tokens(fq):
    rows, cols = W.c3_shape()
    t = time.time()
    cfg = fq.Fp4Config()
    oc = O.Cfg()
    for which in (0, 1):
        xh = W.c3_kv(which)
        x = dev(xh)
        ts = fq.fp4_tensor_scale(x, cfg)
        o_ts = O.tensor_scale(oc, xh)
        assert f32bits(ts.item()) == f32bits(o_ts)
        c, s = fq.fp4_quantize(x, cfg, ts)
        idx = sample_rows(rows, k=64, seed=which)
        check_rows(fq, cfg, O.RTN, xh, c, s, o_ts, idx, tag=f"c3 {which}")
        dq = fq.fp4_dequantize(c, s, cfg, rows, cols, ts, dtype=torch.bfloat16)
        dqh = dq.view(torch.int16).cpu().numpy()
        cn, sn = c.cpu().numpy().reshape(rows, -1), s.cpu().numpy().reshape(rows, -1)
        for r in idx:
            want = O.dequantize(oc, cn[r], sn[r], o_ts, 1, cols, out_bf16=True)
            assert (dqh[r] == want.view(np.int16)).all()
        del x
    say(f"C3 K and V bit-exact on sampled rows ({time.time() - t:.1f} s)")


def test_c4_guidance_cache_layer(fq):
    t = time.time()
    cfg = fq.Fp4Config()
    oc = O.Cfg()
    n_layer = 0
    for name, r, c, sigma, seed, stream in W.c4_tensors(20):
        xh, xrh = W.c4_pair(r, c, sigma, seed, stream)
        n_layer += r * c
        x, xr = dev(xh), dev(xrh)
        ts = fq.fp4_tensor_scale(xr, cfg)
        rc, rs, eb = fq.fp4_quantize(xr, cfg, ts, emit=True)
        gb, gs = fq.guide_pack(rc, rs, cfg, r, c)
        assert torch.equal(gb, eb) and torch.equal(gs, rs)      # fused emission == guide_pack
        gc, gsc = fq.fp4_quantize_guided(x, cfg, gb, gs, ts)
        o_ts = O.tensor_scale(oc, xrh)
        assert f32bits(ts.item()) == f32bits(o_ts)
        idx = sample_rows(r, k=8, seed=stream)
        check_rows(fq, cfg, O.GUIDED, xh, gc, gsc, o_ts, idx, gb=gb.cpu().numpy(), gs=gs.cpu().numpy(),
                   tag=f"c4 {name}")
    guide = 20 * (n_layer // 8 + n_layer // 16)
    full = 40 * (n_layer // 2 + n_layer // 16)
    assert guide == 314_572_800 and full == 1_887_436_800 and 6 * guide == full
    assert fq.guide_bytes(fq.NVFP4, 8192, 4096) == 8192 * 4096 // 8 + 8192 * 4096 // 16 + 4
    say(f"C4 layer bit-exact on sampled rows ({time.time() - t:.1f} s)")


def test_c5_uniform_rht16_sr_65536x8192(fq):
    rows, cols = W.c5_shape()
    t = time.time()
    xh = W.c5_x(rows, cols)
    say(f"C5 generated ({time.time() - t:.1f} s)")
    cfg = fq.Fp4Config(grid=fq.UNIFORM, rounding=fq.SR, rht16=True, rht_seed=W.C5_RHT_SEED,
                       sr_seed=W.C5_SR_SEED)
    oc = O.Cfg(grid=O.UNIFORM, rht16=True, rht_seed=W.C5_RHT_SEED, sr_seed=W.C5_SR_SEED)
    x = dev(xh)
    ts = fq.fp4_tensor_scale(x, cfg)
    c, s = fq.fp4_quantize(x, cfg, ts)
    o_ts = O.tensor_scale(oc, xh)
    say(f"C5 oracle tensor scale ({time.time() - t:.1f} s)")
    assert f32bits(ts.item()) == f32bits(o_ts)
    idx = sample_rows(rows, k=32)
    check_rows(fq, cfg, O.SR, xh, c, s, o_ts, idx, tag="c5")
    say(f"C5 bit-exact on {len(idx)} rows ({time.time() - t:.1f} s)")


@pytest.mark.parametrize("rows", [8191, 8192])
@pytest.mark.parametrize("fmt", [0, 1])
def test_both_slot_counts_at_the_small_launch_threshold(fq, fmt, rows):
    # A single-tensor launch below 2048 workgroups of four slots takes two slots
    # per lane: 8191 x 2048 (NVFP4: 2047 workgroups of four) launches two, 8192 x 2048
    # launches four.  Both equal the oracle in every mode, on the whole tensor.
    cols = 2048
    say("slot threshold", fmt, rows, cols)
    xh = W.c1_x(rows, cols, seed=21)
    xrh = W.c1_rollout(rows, cols, seed=21)
    cfg = fq.Fp4Config(format=fmt)
    oc = O.Cfg(format=fmt)
    x, xr = dev(xh), dev(xrh)
    ts_t = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    ts = O.tensor_scale(oc, xrh) if fmt == 0 else 1.0
    if fmt == 0:
        assert f32bits(ts_t.item()) == f32bits(ts)
    rc, rs, rb = fq.fp4_quantize(xr, cfg, ts_t, emit=True)
    o_rc, o_rs, o_rb = O.quantize(oc, O.RTN, xrh, ts, emit=True)
    assert (rc.cpu().numpy() == o_rc).all() and (rs.cpu().numpy() == o_rs).all()
    assert (rb.cpu().numpy() == o_rb).all()
    gc, gs = fq.fp4_quantize_guided(x, cfg, rb, rs, ts_t)
    o_gc, o_gs = O.quantize(oc, O.GUIDED, xh, ts, guide_bits=o_rb, guide_scales=o_rs)
    assert (gc.cpu().numpy() == o_gc).all() and (gs.cpu().numpy() == o_gs).all()
    scfg = fq.Fp4Config(format=fmt, rounding=fq.SR, sr_seed=5, sr_offset=9)
    sc, ss = fq.fp4_quantize(x, scfg, ts_t)
    o_sc, o_ss = O.quantize(O.Cfg(format=fmt, sr_seed=5, sr_offset=9), O.SR, xh, ts)
    assert (sc.cpu().numpy() == o_sc).all() and (ss.cpu().numpy() == o_ss).all()
