"""GPU parity: every output of the HIP path equals the CPU oracle bit for bit.

Shapes span many workgroups (one workgroup covers 512 groups of 16 elements)
and leave ragged tails; padded row strides, empty inputs and degenerate
blocks are included.  Floating-point outputs (tensor scale, dequantized
values, RHT) are compared as bit patterns: tolerance 0 ulp.
"""
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
    fq_lib = fp4q.lib()
    return fp4q


def dev(u16: np.ndarray, pad: int = 0) -> torch.Tensor:
    """Host bf16 bit patterns -> device bf16 matrix, optionally with padded rows (ld = cols + pad)."""
    rows, cols = u16.shape
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
    if pad:
        buf = torch.full((rows, cols + pad), float("nan"), dtype=torch.bfloat16)
        buf[:, :cols] = t
        return buf.cuda()[:, :cols]
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def ocfg(fqc) -> O.Cfg:
    return O.Cfg(format=fqc.format, grid=fqc.grid, rht16=fqc.rht16, rht_seed=fqc.rht_seed,
                 sr_seed=fqc.sr_seed, sr_offset=fqc.sr_offset)


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


SHAPES = [(256, 512), (37, 544), (1, 32), (129, 96)]


def _data(kind, rows, cols, seed):
    if kind == "normal":
        return W.c1_x(rows, cols, seed=seed)
    if kind == "student":
        return W.c2_pair(rows, cols, seed=seed)[0]
    return W.c5_x(rows, cols, seed=seed)


# ---------------------------------------------------------------- element encode

@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("mode", [0, 1, 2])
def test_encode_values_vs_oracle(fq, grid, mode):
    h = np.arange(0, 0x10000, dtype=np.uint32)
    bfv = (h << 16).view(np.float32)
    bfv = bfv[~np.isnan(bfv)]
    gmax = 6.0 if grid == 0 else 7.0
    near = []
    pts = [0, .25, .5, .75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 6.5, 7, 7.5, 8] + \
          [k + 0.5 for k in range(8)]
    for p in pts:
        u = np.array([p], dtype=np.float32).view(np.uint32)[0]
        d = np.arange(-300, 301, dtype=np.int64) + int(u)
        d = d[d >= 0].astype(np.uint32)
        near.append(d.view(np.float32))
    rng = np.random.default_rng(grid * 3 + mode)
    rnd = rng.uniform(0, gmax + 1, 200_000).astype(np.float32)
    tiny = (rng.uniform(0, 1, 20_000) * 2.0 ** rng.integers(-149, -1, 20_000)).astype(np.float32)
    v = np.concatenate([bfv] + near + [rnd, tiny])
    v = np.concatenate([v, -v])
    v = v[: v.size // 8 * 8]
    if mode == 1:
        aux = rng.integers(0, 256, v.size, dtype=np.uint8)
    elif mode == 2:
        aux = rng.integers(0, 2, v.size, dtype=np.uint8)
    else:
        aux = None
    out = fq.fp4_encode_values(torch.from_numpy(v).cuda(), grid, mode,
                               None if aux is None else torch.from_numpy(aux).cuda())
    got = host(out)
    k = O.encode_many(grid, mode, np.abs(v), None if aux is None else aux.astype(np.uint32))
    want = (np.signbit(v).astype(np.uint8) << 3) | k
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), int(aux[i]) if aux is not None else None, int(got[i]), int(want[i]))
                           for i in bad[:10]]


# ---------------------------------------------------------------- quantize

CASES = [
    # (format, grid, rounding/mode, rht, data)
    (0, 0, 0, False, "normal"),
    (0, 0, 1, False, "normal"),
    (1, 0, 0, False, "student"),
    (1, 0, 1, False, "student"),
    (0, 1, 0, False, "outlier"),
    (0, 1, 1, True, "outlier"),
    (0, 0, 0, True, "outlier"),
    (1, 1, 1, True, "outlier"),
    (1, 0, 0, True, "student"),
    (1, 0, 1, True, "student"),
    (0, 0, 1, True, "outlier"),
    (0, 1, 0, True, "outlier"),
    (0, 1, 1, False, "outlier"),
]


@pytest.mark.parametrize("fmt,grid,rnd,rht,data", CASES)
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("pad", [0, 24])
def test_quantize_vs_oracle(fq, fmt, grid, rnd, rht, data, shape, pad):
    rows, cols = shape
    if cols % (32 if fmt else 16):
        pytest.skip("shape not valid for this block size")
    xh = _data(data, rows, cols, seed=rows + cols)
    cfg = fq.Fp4Config(format=fmt, grid=grid, rounding=rnd, rht16=rht, rht_seed=7, sr_seed=0xABCDEF0123,
                       sr_offset=3)
    oc = ocfg(cfg)
    x = dev(xh, pad)
    ts_t = None
    ts = 1.0
    if fmt == 0:
        ts_t = fq.fp4_tensor_scale(x, cfg)
        ts = O.tensor_scale(oc, xh)
        assert f32_bits(host(ts_t))[0] == f32_bits([ts])[0]
    codes, scales, bits = fq.fp4_quantize(x, cfg, ts_t, emit=True)
    oc_codes, oc_scales, oc_bits = O.quantize(oc, rnd, xh, ts, emit=True)
    assert (host(scales) == oc_scales).all()
    assert (host(codes) == oc_codes).all()
    assert (host(bits) == oc_bits).all()
    # without emission the codes are the same
    c2, s2 = fq.fp4_quantize(x, cfg, ts_t)
    assert (host(c2) == oc_codes).all() and (host(s2) == oc_scales).all()


@pytest.mark.parametrize("fmt,grid,rht", [(0, 0, False), (1, 0, False), (0, 1, False), (1, 1, True), (0, 0, True)])
@pytest.mark.parametrize("shape", SHAPES)
def test_guided_vs_oracle(fq, fmt, grid, rht, shape):
    rows, cols = shape
    if cols % (32 if fmt else 16):
        pytest.skip("shape not valid for this block size")
    x_h = W.c1_x(rows, cols, seed=11)
    xr_h = W.c1_rollout(rows, cols, seed=11)
    cfg = fq.Fp4Config(format=fmt, grid=grid, rht16=rht, rht_seed=7)
    oc = ocfg(cfg)
    xr, x = dev(xr_h), dev(x_h, pad=8)
    ts_t = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    ts = O.tensor_scale(oc, xr_h) if fmt == 0 else 1.0
    rc, rs = fq.fp4_quantize(xr, cfg, ts_t)
    gb, gs = fq.guide_pack(rc, rs, cfg, rows, cols)
    o_rc, o_rs = O.quantize(oc, O.RTN, xr_h, ts)
    o_gb, o_gs = O.guide_pack(oc, o_rc, o_rs, rows, cols)
    assert (host(gb) == o_gb).all() and (host(gs) == o_gs).all()
    gc, gsc = fq.fp4_quantize_guided(x, cfg, gb, gs, ts_t)
    o_gc, o_gsc = O.quantize(oc, O.GUIDED, x_h, ts, guide_bits=o_gb, guide_scales=o_gs)
    assert (host(gsc) == o_gsc).all()
    assert (host(gc) == o_gc).all()
    # the tensor's own RTN guide reproduces RTN bit for bit
    own_c, own_s, own_b = fq.fp4_quantize(x, cfg, ts_t, emit=True)
    g2c, _ = fq.fp4_quantize_guided(x, cfg, own_b, own_s, ts_t)
    assert (host(g2c) == host(own_c)).all()


def test_special_blocks(fq):
    x = np.zeros((2, 96), dtype=np.float32)
    x[0, 16:32] = -0.0
    x[0, 32] = 1000.0
    x[0, 48:64] = np.float32(2.0 ** -130)
    x[0, 64:80] = [0, .5, 1, 1.5, 2, 3, 4, 6, -6, -4, -3, -2, -1.5, -1, -.5, -0.]
    x[1] = np.linspace(-3e38, 3e38, 96)
    xh = W.f32_to_bf16_rne(x)
    xh[0, 85] = 0x7FC0
    xh[0, 90] = 0xFF80
    xh[1, 5] = 0x7F80
    for fmt in (0, 1):
        for rht in (False, True):
            for rnd in (0, 1):
                cfg = fq.Fp4Config(format=fmt, rounding=rnd, rht16=rht, rht_seed=7)
                oc = ocfg(cfg)
                d = dev(xh)
                ts_t = fq.fp4_tensor_scale(d, cfg) if fmt == 0 else None
                ts = O.tensor_scale(oc, xh) if fmt == 0 else 1.0
                if fmt == 0:
                    assert f32_bits(host(ts_t))[0] == f32_bits([ts])[0]
                c, s = fq.fp4_quantize(d, cfg, ts_t)
                oc_c, oc_s = O.quantize(oc, rnd, xh, ts)
                assert (host(s) == oc_s).all(), (fmt, rht, rnd)
                assert (host(c) == oc_c).all(), (fmt, rht, rnd)


@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("ts", [1e35, 3e34, 1.0])
def test_guided_rht_with_tiny_reciprocals(fq, grid, ts):
    # The RHT kernels fold the transform's factor 1/4 into inv unless inv < 2^-124.
    # Guided mode takes block and tensor scales from the caller, so large guide
    # scales with a large tensor scale reach the other branch: S = dec * ts > 2^124.
    rows, cols = 32, 256
    rng = np.random.default_rng(int(ts) % 97 + grid)
    x = (rng.standard_normal((rows, cols)) * 1.5e37).astype(np.float32)
    xh = W.f32_to_bf16_rne(x)
    cfg = fq.Fp4Config(grid=grid, rht16=True, rht_seed=7)
    oc = ocfg(cfg)
    gb = rng.integers(0, 256, rows * cols // 8, dtype=np.uint8)
    gs = rng.choice(np.array([0x7E, 0x7D, 0x76, 0x70, 0x58, 0x38], dtype=np.uint8), rows * cols // 16)
    t32 = np.float32(ts)
    c, s_ = fq.fp4_quantize_guided(dev(xh), cfg, torch.from_numpy(gb).cuda(), torch.from_numpy(gs).cuda(),
                                   torch.tensor([t32], device="cuda"))
    oc_c, oc_s = O.quantize(oc, O.GUIDED, xh, float(t32), guide_bits=gb, guide_scales=gs)
    assert (host(s_) == oc_s).all() and (host(c) == oc_c).all()
    if ts == 1e35:   # the branch is taken for some blocks and the codes are not all zero
        S = np.array([O.e4m3_decode(int(v)) for v in gs]) * float(t32)
        assert (S > 2.0 ** 124).any()
        assert (host(c) != 0).any()


def test_guided_with_nan_guide_scales(fq):
    rows, cols = 8, 64
    xh = W.c1_x(rows, cols, seed=2)
    for fmt in (0, 1):
        cfg = fq.Fp4Config(format=fmt)
        oc = ocfg(cfg)
        rng = np.random.default_rng(fmt)
        gb = rng.integers(0, 256, rows * cols // 8, dtype=np.uint8)
        gs = rng.integers(0, 256, rows * cols // cfg.block, dtype=np.uint8)
        gs[::3] = 0x7F if fmt == 0 else 0xFF
        ts = np.float32(0.0123)
        tst = torch.tensor([ts], device="cuda")
        c, s = fq.fp4_quantize_guided(dev(xh), cfg, torch.from_numpy(gb).cuda(), torch.from_numpy(gs).cuda(), tst)
        oc_c, oc_s = O.quantize(oc, O.GUIDED, xh, float(ts), guide_bits=gb, guide_scales=gs)
        assert (host(s) == oc_s).all() and (host(c) == oc_c).all()


def _midpoint_blocks(rng):
    """bf16 rows of 16-element blocks whose amax is an E4M3 rounding midpoint (1 + (2m+1)/16) 2^e,
    e = -6..8, or one to three bf16 steps either side of it; the other 15 elements are smaller.
    Six more blocks: all zero, amax 2^-7, 2^-6 and its neighbours (the subnormal-code boundary), 448."""
    b6 = int(W.f32_to_bf16_rne(np.array([2.0 ** -6], np.float32))[0])
    amax = [0, b6 - 129, b6 - 1, b6, b6 + 1, 0x43E0]
    for e in range(-6, 9):
        for m in range(8):
            mid = (1 + (2 * m + 1) / 16) * 2.0 ** e
            if mid > 448:
                continue
            b = int(W.f32_to_bf16_rne(np.array([mid], np.float32))[0])
            amax += [b + d for d in (-3, -2, -1, 0, 1, 2, 3)]
    amax = np.array(amax, np.uint16)
    blocks = W.f32_to_bf16_rne((rng.uniform(-1, 1, (len(amax), 16)) *
                                W.bf16_to_f32(amax)[:, None] * 0.9).astype(np.float32))
    blocks[np.arange(len(amax)), rng.integers(0, 16, len(amax))] = amax | (rng.integers(0, 2, len(amax)) << 15).astype(np.uint16)
    return blocks.reshape(-1, 64)


# denominators RN(6 s_t) = 1 + k 2^-23 or 1 - k 2^-24: the quotients amax / denom then lie on, or a
# few fp32 steps below or above, the E4M3 midpoints, where the scale code must come from the exact
# quotient (ties to even at the midpoint itself)
@pytest.mark.parametrize("k", [0, 1, 2, 3, 5, -1, -2, -3, -5])
@pytest.mark.parametrize("rnd", [0, 1])
def test_nvfp4_scale_quotient_near_e4m3_midpoints(fq, k, rnd):
    denom = np.float32(1 + k * 2.0 ** -23) if k >= 0 else np.float32(1 + k * 2.0 ** -24)
    ts = np.float32(denom / np.float32(6))
    assert np.float32(6) * ts == denom or k != 0
    xh = _midpoint_blocks(np.random.default_rng(40 + k))
    cfg = fq.Fp4Config(rounding=rnd, sr_seed=5)
    oc = ocfg(cfg)
    c, s = fq.fp4_quantize(dev(xh), cfg, torch.tensor([ts], device="cuda"))
    oc_c, oc_s = O.quantize(oc, rnd, xh, float(ts))
    bad = np.nonzero(host(s) != oc_s)[0]
    assert bad.size == 0, [(int(i), int(host(s)[i]), int(oc_s[i])) for i in bad[:8]]
    assert (host(c) == oc_c).all()


@pytest.mark.parametrize("ts", [1.0, 0.37, 1e-3, 2.0 ** -120, 7.5e37 / 2688, 2.0 ** -128, 1e37])
@pytest.mark.parametrize("rnd", [0, 1])
def test_nvfp4_extreme_tensor_scales(fq, ts, rnd):
    # 1e-38 rows at ts = 2^-120: block scales S below 2^-128, where 1/S saturates to FLT_MAX
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, 64)) * rng.choice([1e-38, 1e-30, 1e-3, 1, 1e3], (16, 1))).astype(np.float32)
    xh = W.f32_to_bf16_rne(x)
    cfg = fq.Fp4Config(rounding=rnd, sr_seed=21)
    oc = ocfg(cfg)
    ts = np.float32(ts)
    tst = torch.tensor([ts], device="cuda")
    c, s = fq.fp4_quantize(dev(xh), cfg, tst)
    oc_c, oc_s = O.quantize(oc, rnd, xh, float(ts))
    assert (host(s) == oc_s).all() and (host(c) == oc_c).all()
    fqo = fq.fp4_fake_quantize(dev(xh), cfg, tst)
    want = O.dequantize(oc, oc_c, oc_s, float(ts), 16, 64, out_bf16=True)
    assert (host(fqo.view(torch.int16)).reshape(-1) == want.view(np.int16)).all()


def test_mxfp4_sr_every_8bit_scaled_value(fq):
    # MXFP4 SR of E2M1 without the RHT runs through the hardware stochastic
    # convert, exact for scaled values with at most 14 significant bits.  Every
    # block gets an anchor 6*2^s (so e = s and v = |y|/2^s) and 31 values from
    # the list of all 8-bit significands times 2^E, E = -11..2, both signs.  Over
    # 4096 rows each value meets each random byte with probability 1 - 1e-7.
    sig = 1.0 + np.arange(128) / 128.0
    vals = np.concatenate([sig * 2.0 ** E for E in range(-11, 3)] + [[0.0, 0.5, 1.5, 3.0, 6.0]])
    vals = np.concatenate([vals, -vals]).astype(np.float64)
    per_row = 31 * ((vals.size + 30) // 31)
    nblk = per_row // 31
    rows, cols = 4096, 32 * nblk
    rng = np.random.default_rng(17)
    x = np.empty((rows, cols), dtype=np.float32)
    for r in range(rows):
        s = (r % 9) - 4
        payload = np.resize(np.roll(vals, r * 7), per_row).reshape(nblk, 31)
        blk = np.empty((nblk, 32))
        blk[:, 0] = 6.0 * (1 if r % 2 else -1)
        blk[:, 1:] = payload
        x[r] = (blk * 2.0 ** s).reshape(-1)
    xh = W.f32_to_bf16_rne(x)
    assert (W.bf16_to_f32(xh) == x).all()       # exact: 8 significant bits
    cfg = fq.Fp4Config(format=1, rounding=1, sr_seed=0x5EED, sr_offset=11)
    oc = ocfg(cfg)
    c, sc = fq.fp4_quantize(dev(xh), cfg)
    oc_c, oc_s = O.quantize(oc, O.SR, xh)
    assert (host(sc) == oc_s).all()
    assert (host(c) == oc_c).all()


@pytest.mark.parametrize("grid", [0, 1])
@pytest.mark.parametrize("rnd", [0, 1])
def test_mxfp4_extreme_magnitudes(fq, grid, rnd):
    rng = np.random.default_rng(11)
    mags = np.float32([2.0 ** -133, 2.0 ** -130, 2.0 ** -127, 2.0 ** -125, 1e-30, 1.0, 1e30, 3.0e38])
    x = (rng.uniform(-1, 1, (8, 64)) * mags[:, None]).astype(np.float32)
    x[:, 0] = mags
    xh = W.f32_to_bf16_rne(x)
    cfg = fq.Fp4Config(format=1, grid=grid, rounding=rnd, sr_seed=4)
    oc = ocfg(cfg)
    c, s = fq.fp4_quantize(dev(xh), cfg)
    oc_c, oc_s = O.quantize(oc, rnd, xh)
    assert oc_s[0] == 0
    assert (host(s) == oc_s).all() and (host(c) == oc_c).all()
    fqo = fq.fp4_fake_quantize(dev(xh), cfg)
    want = O.dequantize(oc, oc_c, oc_s, 1.0, 8, 64, out_bf16=True)
    assert (host(fqo.view(torch.int16)).reshape(-1) == want.view(np.int16)).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_guided_with_a_rescaled_rollout(fq, fmt):
    # the rollout is 1.7x the tensor, so most guide block scales differ from the tensor's own
    rows, cols = 96, 512
    x_h = W.c5_x(rows, cols, seed=6)
    xr_h = W.f32_to_bf16_rne(W.bf16_to_f32(x_h) * np.float32(1.7))
    cfg = fq.Fp4Config(format=fmt)
    oc = ocfg(cfg)
    xr = dev(xr_h)
    ts_t = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    ts = O.tensor_scale(oc, xr_h) if fmt == 0 else 1.0
    _, rs, rb = fq.fp4_quantize(xr, cfg, ts_t, emit=True)
    o_rc, o_rs, o_rb = O.quantize(oc, O.RTN, xr_h, ts, emit=True)
    assert (host(rs) == o_rs).all() and (host(rb) == o_rb).all()
    gc, gsc = fq.fp4_quantize_guided(dev(x_h), cfg, rb, rs, ts_t)
    o_gc, o_gsc = O.quantize(oc, O.GUIDED, x_h, ts, guide_bits=o_rb, guide_scales=o_rs)
    assert (host(gsc) == o_gsc).all() and (host(gc) == o_gc).all()
    fqo = fq.fp4_fake_quantize(dev(x_h), cfg, ts_t, rb, rs)
    want = O.dequantize(oc, o_gc, o_gsc, ts, rows, cols, out_bf16=True)
    assert (host(fqo.view(torch.int16)).reshape(-1) == want.view(np.int16)).all()


def test_dequant_bf16_ties(fq):
    codes = np.arange(256, dtype=np.uint8)
    cfg = fq.Fp4Config()
    oc = ocfg(cfg)
    sc = np.full(32, 0x38, dtype=np.uint8)
    for ts in (1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8):
        ts = np.float32(ts)
        want = O.dequantize(oc, codes, sc, float(ts), 1, 512, out_bf16=True)
        got = fq.fp4_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(sc).cuda(), cfg, 1, 512,
                                torch.tensor([ts], device="cuda"), dtype=torch.bfloat16)
        assert (host(got.view(torch.int16)).reshape(-1) == want.view(np.int16)).all()


@pytest.mark.parametrize("fmt,grid,rht", [(0, 0, False), (1, 0, False), (0, 1, True), (1, 1, True), (1, 0, True)])
@pytest.mark.parametrize("shape,pad", [((256, 512), 0), ((37, 544), 24), ((3, 32), 0), ((129, 96), 8)])
def test_guide_mismatch_vs_oracle(fq, fmt, grid, rht, shape, pad):
    rows, cols = shape
    if cols % (32 if fmt else 16):
        pytest.skip("shape not valid for this block size")
    x_h = W.c1_x(rows, cols, seed=rows + 1)
    xr_h = W.c1_rollout(rows, cols, seed=rows + 1)
    xr_h[::3] = W.f32_to_bf16_rne(W.bf16_to_f32(x_h[::3]) * np.float32(1.7))   # far rollout rows
    cfg = fq.Fp4Config(format=fmt, grid=grid, rht16=rht, rht_seed=7)
    oc = ocfg(cfg)
    xr = dev(xr_h)
    ts_t = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    ts = O.tensor_scale(oc, xr_h) if fmt == 0 else 1.0
    rc, rs = fq.fp4_quantize(xr, cfg, ts_t)
    o_rc, o_rs = O.quantize(oc, O.RTN, xr_h, ts)
    assert (host(rc) == o_rc).all() and (host(rs) == o_rs).all()
    counts = fq.fp4_guide_mismatch(dev(x_h, pad), cfg, rc, rs, ts_t)
    want = O.guide_mismatch(oc, x_h, ts, o_rc, o_rs)
    assert tuple(int(v) for v in host(counts)) == want
    assert want[1] > 0


@pytest.mark.parametrize("fmt,grid,rht", [(0, 1, True), (1, 0, True), (0, 0, False)])
def test_guide_mismatch_several_chunks_per_workgroup(fq, fmt, grid, rht):
    # More chunks than the diagnostic's 1024 workgroups: each workgroup walks
    # several, reusing its LDS (the RHT transpose) and its counters.
    rows, cols = 1088, 8192   # 557,056 groups: 1088 chunks of 512
    x_h = W.c1_x(rows, cols, seed=3)
    xr_h = W.c1_rollout(rows, cols, seed=3)
    xr_h[::5] = W.f32_to_bf16_rne(W.bf16_to_f32(x_h[::5]) * np.float32(1.7))
    cfg = fq.Fp4Config(format=fmt, grid=grid, rht16=rht, rht_seed=7)
    oc = ocfg(cfg)
    xr = dev(xr_h)
    ts_t = fq.fp4_tensor_scale(xr, cfg) if fmt == 0 else None
    ts = O.tensor_scale(oc, xr_h) if fmt == 0 else 1.0
    rc, rs = fq.fp4_quantize(xr, cfg, ts_t)
    o_rc, o_rs = O.quantize(oc, O.RTN, xr_h, ts)
    assert (host(rc) == o_rc).all() and (host(rs) == o_rs).all()
    counts = fq.fp4_guide_mismatch(dev(x_h), cfg, rc, rs, ts_t)
    want = O.guide_mismatch(oc, x_h, ts, o_rc, o_rs)
    assert tuple(int(v) for v in host(counts)) == want
    assert want[1] > 0


def test_guide_mismatch_bracket_cases_and_empty(fq):
    cases = [(2.4, 5), (2.4, 6), (2.4, 0xD), (2.0, 5), (2.0, 4), (-0.3, 9), (0.3, 8), (7.0, 6)] + [(1.0, 2)] * 8
    x = np.array([[v for v, _ in cases] * 3], dtype=np.float32)
    r = np.array([c for _, c in cases] * 3, dtype=np.uint8)
    xh = W.f32_to_bf16_rne(x)
    xh[0, 16 + 3] = 0x7FC0                                   # second block: non-finite input
    rc = (r[0::2] | (r[1::2] << 4)).astype(np.uint8)
    rs = np.array([0x38, 0x38, 0x7F], dtype=np.uint8)        # third block: NaN rollout scale
    cfg = fq.Fp4Config()
    ts = torch.ones(1, device="cuda")
    counts = fq.fp4_guide_mismatch(dev(xh), cfg, torch.from_numpy(rc).cuda(), torch.from_numpy(rs).cuda(), ts)
    assert tuple(int(v) for v in host(counts)) == O.guide_mismatch(O.Cfg(), xh, 1.0, rc, rs) == (16, 3, 5)
    empty = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    out = torch.full((3,), 7, dtype=torch.int64, device="cuda")
    fq.fp4_guide_mismatch(empty, cfg, torch.empty(0, dtype=torch.uint8, device="cuda"),
                          torch.empty(0, dtype=torch.uint8, device="cuda"), ts, out=out)
    assert host(out).tolist() == [0, 0, 0]


# ---------------------------------------------------------------- dequantize, guide, rht

@pytest.mark.parametrize("fmt,grid", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("shape", [(256, 512), (37, 544), (3, 32), (5, 48), (1, 16), (300, 2080), (777, 1040)])
def test_dequantize_vs_oracle(fq, fmt, grid, shape):
    rows, cols = shape
    B = 32 if fmt else 16
    if cols % B:
        pytest.skip("shape not valid for this block size")
    rng = np.random.default_rng(rows)
    codes = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    scales = rng.integers(0, 256, rows * cols // B, dtype=np.uint8)
    ts = np.float32(rng.uniform(1e-4, 3.0))
    cfg = fq.Fp4Config(format=fmt, grid=grid)
    oc = ocfg(cfg)
    ct, st = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    tst = torch.tensor([ts], device="cuda")
    for bf16 in (False, True):
        want = O.dequantize(oc, codes, scales, float(ts), rows, cols, out_bf16=bf16)
        dt = torch.bfloat16 if bf16 else torch.float32
        got = fq.fp4_dequantize(ct, st, cfg, rows, cols, tst, dtype=dt)
        g = host(got.view(torch.int16) if bf16 else got.view(torch.int32)).reshape(-1)
        w = want.view(np.int16 if bf16 else np.int32)
        assert (g == w).all(), (bf16, np.nonzero(g != w)[0][:5])
        # padded output rows
        out = torch.zeros((rows, cols + 64), dtype=dt, device="cuda")[:, :cols]
        fq.fp4_dequantize(ct, st, cfg, rows, cols, tst, out=out)
        g2 = host(out.contiguous().view(torch.int16) if bf16 else out.contiguous().view(torch.int32)).reshape(-1)
        assert (g2 == w).all()


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("shape", [(77, 544), (5, 48), (1, 16), (3, 16), (300, 2080)])
def test_guide_pack_unpack_vs_oracle(fq, fmt, shape):
    rows, cols = shape
    B = 32 if fmt else 16
    if cols % B:
        pytest.skip("shape not valid for this block size")
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, rows * cols // 2, dtype=np.uint8)
    scales = rng.integers(0, 256, rows * cols // B, dtype=np.uint8)
    cfg = fq.Fp4Config(format=fmt)
    oc = ocfg(cfg)
    gb, gs = fq.guide_pack(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), cfg, rows, cols)
    o_gb, o_gs = O.guide_pack(oc, codes, scales, rows, cols)
    assert (host(gb) == o_gb).all() and (host(gs) == o_gs).all()
    m, so = fq.guide_unpack(gb, gs, cfg, rows, cols)
    o_m, o_so = O.guide_unpack(oc, o_gb, o_gs, rows, cols)
    assert (host(m) == o_m).all() and (host(so) == o_so).all()
    # scale arrays at odd addresses (the ABI asks for byte alignment only)
    sbuf = torch.zeros(scales.size + 1, dtype=torch.uint8, device="cuda")
    sbuf[1:] = torch.from_numpy(scales).cuda()
    gsbuf = torch.full((scales.size + 3,), 0xA5, dtype=torch.uint8, device="cuda")
    gb2, gs2 = fq.guide_pack(torch.from_numpy(codes).cuda(), sbuf[1:], cfg, rows, cols,
                             gscales=gsbuf[3:])
    assert (host(gb2) == o_gb).all() and (host(gs2) == o_gs).all()
    assert (host(gsbuf[:3]) == 0xA5).all()


@pytest.mark.parametrize("inverse", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("pad", [0, 40])
def test_rht16_vs_oracle(fq, inverse, bf16, pad):
    rows, cols = 133, 256
    xh = W.c5_x(rows, cols, seed=9)
    out = fq.fp4_rht16(dev(xh, pad), 7, inverse=inverse, dtype=torch.bfloat16 if bf16 else torch.float32)
    want = O.rht16(xh, 7, inverse=inverse, out_bf16=bf16)
    g = host(out.view(torch.int16) if bf16 else out.view(torch.int32)).reshape(-1)
    assert (g == want.view(np.int16 if bf16 else np.int32)).all()


@pytest.mark.parametrize("rht", [False, True])
@pytest.mark.parametrize("shape,pad", [((3, 16), 0), ((5, 48), 8), ((129, 96), 0), ((1, 16 * 1027), 0)])
def test_tensor_scale_ragged_tail(fq, rht, shape, pad):
    # Lanes past the end of the tensor read its last half-group (8 elements)
    # again.  Here the last group is 8 zeros and then the only large values, so
    # that half-group doubled would transform to a larger maximum than any real
    # group: the tensor scale must come from real groups only.
    rows, cols = shape
    rng = np.random.default_rng(rows * cols)
    xf = (rng.standard_normal((rows, cols)) * 1e-3).astype(np.float32)
    xf[-1, -16:-8] = 0.0
    xf[-1, -8:] = 3.0
    xh = W.f32_to_bf16_rne(xf)
    cfg = fq.Fp4Config(rht16=rht, rht_seed=7)
    oc = ocfg(cfg)
    if rht:   # the doubled half-group would indeed give a larger amax than the real last group
        real = O.rht16(xh[-1:, -16:], 7)
        fake = O.rht16(np.concatenate([xh[-1, -8:], xh[-1, -8:]])[None, :], 7)
        assert np.abs(fake).max() > np.abs(real).max()
    ts = fq.fp4_tensor_scale(dev(xh, pad), cfg)
    assert f32_bits(host(ts))[0] == f32_bits([O.tensor_scale(oc, xh)])[0]


def test_empty_inputs(fq):
    cfg = fq.Fp4Config()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ts = fq.fp4_tensor_scale(x, cfg)
    assert host(ts)[0] == 1.0
    c, s = fq.fp4_quantize(x, cfg, ts)
    assert c.numel() == 0 and s.numel() == 0
