"""Tensor-level pins for the oracle (CPU).

* NVFP4 block scale, element encode and packing are recomputed with an
  independent pipeline: torch float32 arithmetic (IEEE, correctly rounded),
  torch's float8_e4m3fn cast for the scale, brute-force nearest codeword.
* MXFP4 scale exponent from numpy's frexp.
* guided with the tensor's own RTN guide reproduces RTN bit for bit; guided
  output always sits in the bracket and carries the guide bit.
* Stochastic rounding's random bytes come from Philox at the group index;
  rows quantized on their own match the same rows of the whole tensor.
* Dequantization equals the exact product rounded once (0 ulp).
* Degenerate blocks: zero, signed zero, single outlier, subnormals, on-grid
  values, non-finite values.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import to_f32
from precision_rl_amd import workloads as W

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
UNIF = np.arange(8, dtype=np.float64)


def _grid(g):
    return E2M1 if g == 0 else UNIF


def _bf16(a):
    return W.f32_to_bf16_rne(np.asarray(a, dtype=np.float32))


def _f32(h):
    return W.bf16_to_f32(h)


def _nearest_even(vc, G):
    d = np.abs(vc[..., None] - G)
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8) % 2 == 0)
    return np.where(even.any(-1), even.argmax(-1), cand.argmax(-1))


def _pack(code):
    code = code.reshape(-1).astype(np.uint8)
    return (code[0::2] | (code[1::2] << 4)).astype(np.uint8)


def _unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out


def torch_nvfp4_rtn(xh, ts, grid=0):
    """Independent NVFP4 RTN: torch float32 ops + torch E4M3 cast + brute-force nearest."""
    R, C = xh.shape
    G = _grid(grid)
    x = torch.from_numpy(_f32(xh).reshape(R, C // 16, 16).copy())
    ts_t = torch.tensor(ts, dtype=torch.float32)
    amax = x.abs().amax(-1)
    denom = torch.tensor(float(G[-1]), dtype=torch.float32) * ts_t
    t = amax / denom
    code = t.clamp(max=448.0).to(torch.float8_e4m3fn)
    d = code.to(torch.float32)
    S = d * ts_t
    inv = torch.where(S == 0, torch.zeros_like(S), 1.0 / S)
    inv = torch.where(torch.isinf(inv), torch.full_like(inv, np.finfo(np.float32).max), inv)
    v = (x.abs() * inv[..., None]).numpy().astype(np.float64)
    k = _nearest_even(np.minimum(v, G[-1]), G)
    sign = np.signbit(x.numpy()).astype(np.int64)
    codes = (sign << 3) | k
    return _pack(codes), code.view(torch.uint8).numpy().reshape(-1)


def numpy_mxfp4_rtn(xh, grid=0):
    R, C = xh.shape
    G = _grid(grid)
    x = _f32(xh).reshape(R, C // 32, 32)
    amax = np.abs(x).max(-1).astype(np.float64)
    _, ex = np.frexp(amax)
    e = np.where(amax == 0, -127, np.clip(ex - 1 - 2, -127, 127))
    inv = np.ldexp(np.float32(1.0), -e).astype(np.float32)
    v = (np.abs(x) * inv[..., None]).astype(np.float32).astype(np.float64)
    k = _nearest_even(np.minimum(v, G[-1]), G)
    codes = (np.signbit(x).astype(np.int64) << 3) | k
    return _pack(codes), (e + 127).astype(np.uint8).reshape(-1)


@pytest.mark.parametrize("grid", [0, 1])
def test_nvfp4_rtn_matches_independent_pipeline(orc, grid):
    R, C = 64, 256
    xh = W.c1_x(R, C, seed=5)
    cfg = orc.Cfg(format=orc.NVFP4, grid=grid)
    ts = orc.tensor_scale(cfg, xh)
    codes, scales = orc.quantize(cfg, orc.RTN, xh, ts)
    rc, rs = torch_nvfp4_rtn(xh, ts, grid)
    assert (scales == rs).all()
    assert (codes == rc).all()


@pytest.mark.parametrize("ts", [1.0, 0.37, 1e-3, 2.0 ** -120, 7.5e37 / 2688])
def test_nvfp4_scale_rule_at_extreme_tensor_scales(orc, ts):
    rng = np.random.default_rng(9)
    # 1e-38 rows at ts = 2^-120 give block scales S = d*ts below 2^-128, where 1/S overflows
    x = (rng.standard_normal((16, 64)) * rng.choice([1e-38, 1e-30, 1e-3, 1, 1e3], (16, 1))).astype(np.float32)
    xh = _bf16(x)
    cfg = orc.Cfg(format=orc.NVFP4)
    codes, scales = orc.quantize(cfg, orc.RTN, xh, np.float32(ts))
    rc, rs = torch_nvfp4_rtn(xh, float(np.float32(ts)))
    assert (scales == rs).all() and (codes == rc).all()


@pytest.mark.parametrize("grid", [0, 1])
def test_mxfp4_rtn_matches_frexp_pipeline(orc, grid):
    xh, _ = W.c2_pair(64, 256, seed=4)
    cfg = orc.Cfg(format=orc.MXFP4, grid=grid)
    codes, scales = orc.quantize(cfg, orc.RTN, xh)
    rc, rs = numpy_mxfp4_rtn(xh, grid)
    assert (scales == rs).all() and (codes == rc).all()


@pytest.mark.parametrize("grid", [0, 1])
def test_mxfp4_rtn_at_extreme_magnitudes(orc, grid):
    # block amax from the smallest bf16 subnormal (2^-133, exponent clamped at -127)
    # up to the largest finite bf16 value
    rng = np.random.default_rng(11)
    mags = np.float32([2.0 ** -133, 2.0 ** -130, 2.0 ** -127, 2.0 ** -125, 1e-30, 1.0, 1e30, 3.0e38])
    x = (rng.uniform(-1, 1, (8, 64)) * mags[:, None]).astype(np.float32)
    x[:, 0] = mags  # each row's amax is its magnitude
    xh = _bf16(x)
    cfg = orc.Cfg(format=orc.MXFP4, grid=grid)
    codes, scales = orc.quantize(cfg, orc.RTN, xh)
    rc, rs = numpy_mxfp4_rtn(xh, grid)
    assert (scales == rs).all() and (codes == rc).all()
    assert scales[0] == 0 and scales[-1] == 125 + 127


def test_tensor_scale_is_amax_over_2688(orc):
    xh = W.c1_x(128, 512, seed=3)
    amax = np.abs(_f32(xh)).max()
    assert orc.tensor_scale(orc.Cfg(), xh) == np.float32(amax) / np.float32(2688.0)
    assert orc.tensor_scale(orc.Cfg(grid=1), xh) == np.float32(amax) / np.float32(3136.0)
    assert orc.tensor_scale(orc.Cfg(), np.zeros((4, 16), dtype=np.uint16)) == 1.0
    # non-finite values are skipped
    y = xh.copy()
    y[0, 0] = 0x7F80
    y[1, 3] = 0xFFC0
    amax2 = np.abs(np.where(np.isfinite(_f32(y)), _f32(y), 0)).max()
    assert orc.tensor_scale(orc.Cfg(), y) == np.float32(amax2) / np.float32(2688.0)


@pytest.mark.parametrize("fmt,grid,rht", [(0, 0, False), (1, 0, False), (0, 1, True), (1, 1, False), (0, 0, True)])
def test_guided_with_own_rtn_guide_reproduces_rtn(orc, fmt, grid, rht):
    xh = W.c5_x(32, 512, seed=2)
    cfg = orc.Cfg(format=fmt, grid=grid, rht16=rht, rht_seed=7)
    ts = orc.tensor_scale(cfg, xh)
    codes, scales, bits = orc.quantize(cfg, orc.RTN, xh, ts, emit=True)
    gb, gs = orc.guide_pack(cfg, codes, scales, 32, 512)
    assert (gb == bits).all() and (gs == scales).all()
    g_codes, g_scales = orc.quantize(cfg, orc.GUIDED, xh, ts, guide_bits=gb, guide_scales=gs)
    assert (g_codes == codes).all() and (g_scales == scales).all()


def test_guided_invariants_against_a_perturbed_rollout(orc):
    R, C = 64, 512
    x = W.c1_x(R, C, seed=1)
    xr = W.c1_rollout(R, C, seed=1)
    cfg = orc.Cfg()
    ts_r = orc.tensor_scale(cfg, xr)
    rc, rs = orc.quantize(cfg, orc.RTN, xr, ts_r)
    gb, gs = orc.guide_pack(cfg, rc, rs, R, C)
    gc, gsc = orc.quantize(cfg, orc.GUIDED, x, ts_r, guide_bits=gb, guide_scales=gs)
    assert (gsc == rs).all()
    # recompute the bracket of every element with the guide's scale (torch float32)
    xf = torch.from_numpy(_f32(x).reshape(R, C // 16, 16).copy())
    d = torch.from_numpy(gs.copy()).view(torch.float8_e4m3fn).to(torch.float32).reshape(R, C // 16)
    S = d * torch.tensor(ts_r, dtype=torch.float32)
    inv = torch.where(S == 0, torch.zeros_like(S), 1.0 / S)
    v = np.minimum((xf.abs() * inv[..., None]).numpy().astype(np.float64).reshape(-1), 6.0)
    klo = np.searchsorted(E2M1, v, side="right") - 1
    khi = np.searchsorted(E2M1, v, side="left")
    k = (_unpack(gc) & 7).astype(int)
    bit = np.unpackbits(gb, bitorder="little").astype(int)
    assert ((k == klo) | (k == khi)).all()
    off = klo != khi
    assert ((k[off] & 1) == bit[off]).all()
    # mismatch diagnostic: guided agrees with the rollout codeword far more than RTN does
    rk = _unpack(rc) & 7
    own, _ = orc.quantize(cfg, orc.RTN, x, ts_r)
    ok = _unpack(own) & 7
    assert (k == rk).mean() >= (ok == rk).mean()


def test_guided_takes_block_scales_from_the_guide(orc):
    # the rollout is the tensor scaled by 1.7 (bf16), so its block scales differ from
    # the ones the tensor would get on its own; guided output must keep the guide's
    R, C = 32, 256
    x = W.c5_x(R, C, seed=6)
    xr = _bf16(_f32(x) * np.float32(1.7))
    for fmt in (orc.NVFP4, orc.MXFP4):
        cfg = orc.Cfg(format=fmt)
        B = cfg.block
        ts = orc.tensor_scale(cfg, xr) if fmt == orc.NVFP4 else 1.0
        rc, rs = orc.quantize(cfg, orc.RTN, xr, ts)
        own_c, own_s = orc.quantize(cfg, orc.RTN, x, ts)
        assert (own_s != rs).mean() > 0.5
        gb, gs = orc.guide_pack(cfg, rc, rs, R, C)
        gc, gsc = orc.quantize(cfg, orc.GUIDED, x, ts, guide_bits=gb, guide_scales=gs)
        assert (gsc == rs).all()
        xf = torch.from_numpy(_f32(x).reshape(R, C // B, B).copy())
        if fmt == orc.NVFP4:
            d = torch.from_numpy(gs.copy()).view(torch.float8_e4m3fn).to(torch.float32).reshape(R, C // B)
            S = d * torch.tensor(ts, dtype=torch.float32)
            inv = torch.where(S == 0, torch.zeros_like(S), 1.0 / S)
        else:
            e = torch.from_numpy(gs.astype(np.int64)).reshape(R, C // B) - 127
            inv = torch.pow(2.0, -e.to(torch.float64)).to(torch.float32)
        v = np.minimum((xf.abs() * inv[..., None]).numpy().astype(np.float64).reshape(-1), 6.0)
        klo = np.searchsorted(E2M1, v, side="right") - 1
        khi = np.searchsorted(E2M1, v, side="left")
        k = (_unpack(gc) & 7).astype(int)
        bit = np.unpackbits(gb, bitorder="little").astype(int)
        assert ((k == klo) | (k == khi)).all()
        assert ((k[klo != khi] & 1) == bit[klo != khi]).all()


def test_guided_nan_guide_scale_gives_zero_codes(orc):
    # E4M3FN NaN is S.1111.111 (0x7F and 0xFF); E8M0 NaN is 0xFF
    R, C = 1, 128
    x = _bf16(np.linspace(-5, 5, C, dtype=np.float32)[None, :])
    gb = np.full(C // 8, 0xFF, dtype=np.uint8)  # guide bit 1 everywhere: never the zero code
    gs = np.array([0x7F, 0x38, 0xFF, 0x38, 0x40, 0x7F, 0x30, 0xFF], dtype=np.uint8)
    cfg = orc.Cfg()
    gc, gsc = orc.quantize(cfg, orc.GUIDED, x, 1.0, guide_bits=gb, guide_scales=gs)
    nib = _unpack(gc).reshape(8, 16)
    assert (gsc == gs).all()
    for b in range(8):
        nan = gs[b] & 0x7F == 0x7F
        assert (nib[b] == 0).all() == nan, b
    cfgm = orc.Cfg(format=orc.MXFP4)
    gsm = np.array([0xFF, 127, 0xFE, 0xFF], dtype=np.uint8)
    gc, gsc = orc.quantize(cfgm, orc.GUIDED, x, 1.0, guide_bits=gb, guide_scales=gsm)
    nib = _unpack(gc).reshape(4, 32)
    assert (gsc == gsm).all()
    assert (nib[0] == 0).all() and (nib[3] == 0).all() and (nib[1] != 0).any()


def test_sr_random_bytes_follow_the_group_counter(orc):
    R, C = 8, 64
    xh = W.c5_x(R, C, seed=3)
    seed, off = 0x1234_5678_9ABC, 17
    cfg = orc.Cfg(format=orc.MXFP4, sr_seed=seed, sr_offset=off)
    codes, scales = orc.quantize(cfg, orc.SR, xh)
    x = _f32(xh).reshape(-1)
    e = scales.astype(int) - 127
    inv = np.ldexp(np.float32(1.0), -np.repeat(e, 32)).astype(np.float32)
    v = np.minimum((np.abs(x) * inv).astype(np.float64), 6.0)
    n = x.size
    u = np.empty(n, dtype=np.int64)
    for g in range(n // 16):
        ctr = g + off
        w = orc.philox4x32_10((ctr & 0xFFFFFFFF, ctr >> 32, 0, 0), (seed & 0xFFFFFFFF, seed >> 32))
        u[16 * g:16 * g + 16] = np.frombuffer(np.array(w, dtype=np.uint32).tobytes(), dtype=np.uint8)
    klo = np.searchsorted(E2M1, v, side="right") - 1
    khi = np.searchsorted(E2M1, v, side="left")
    f = np.where(khi > klo, (v - E2M1[klo]) / np.where(khi > klo, E2M1[khi] - E2M1[klo], 1), 0)
    up = (2 * u + 1) < 512 * f
    k = np.where(up, khi, klo)
    want = (np.signbit(x).astype(int) << 3) | k
    assert (_unpack(codes) == want).all()


@pytest.mark.parametrize("mode", [0, 1])
def test_row_subset_matches_whole_tensor(orc, mode):
    R, C = 40, 96
    xh = W.c5_x(R, C, seed=4)
    cfg = orc.Cfg(format=orc.NVFP4, sr_seed=3, sr_offset=5)
    ts = orc.tensor_scale(cfg, xh)
    full_c, full_s = orc.quantize(cfg, mode, xh, ts)
    part_c, part_s = orc.quantize(cfg, mode, xh[13:29], ts, row0=13)
    assert (part_c == full_c[13 * C // 2: 29 * C // 2]).all()
    assert (part_s == full_s[13 * C // 16: 29 * C // 16]).all()
    # padded rows (ld > cols) give the same result as dense rows
    pad = np.zeros((R, C + 32), dtype=np.uint16)
    pad[:, :C] = xh
    pad[:, C:] = 0x7F80  # garbage beyond cols must be ignored
    pc, ps = orc.quantize(cfg, mode, pad, ts, cols=C)
    assert (pc == full_c).all() and (ps == full_s).all()


def test_sr_is_unbiased_over_seeds(orc):
    rng = np.random.default_rng(0)
    x = rng.uniform(-5, 5, (1, 64)).astype(np.float32)
    x[0, :16] *= 1e-2
    xh = _bf16(x)
    cfg0 = orc.Cfg(format=orc.MXFP4)
    _, scales = orc.quantize(cfg0, orc.RTN, xh)
    acc = np.zeros(64)
    n = 3000
    for s in range(n):
        cfg = orc.Cfg(format=orc.MXFP4, sr_seed=s)
        c, sc = orc.quantize(cfg, orc.SR, xh)
        assert (sc == scales).all()
        acc += orc.dequantize(cfg, c, sc, 1.0, 1, 64)
    mean = acc / n
    xv = _f32(xh).reshape(-1).astype(np.float64)
    e = np.repeat(scales.astype(int) - 127, 32)
    gap = np.ldexp(2.0, e)  # widest step of the grid at this scale
    # per-element SR variance <= gap^2/4: mean within 5 sigma + the 2^-9 bias bound
    assert (np.abs(mean - xv) <= 5 * gap / 2 / np.sqrt(n) + gap / 512).all()


def test_dequant_is_exact_product_rounded_once(orc):
    rng = np.random.default_rng(4)
    codes = np.arange(256, dtype=np.uint8).reshape(16, 16).reshape(-1)  # every code pair
    for ts in [1.0, 0.3333, 2.0 ** -126 * 3, 1.7e-5, 1e30]:
        ts = float(np.float32(ts))
        scodes = rng.integers(0, 0x7F, 32).astype(np.uint8)
        cfg = orc.Cfg()
        out = orc.dequantize(cfg, codes, scodes, ts, 1, 512)
        nib = _unpack(codes)
        for i in range(512):
            c = int(nib[i])
            s = int(scodes[i // 16])
            d = Fraction(orc.e4m3_decode(s))
            g = Fraction(float(E2M1[c & 7]))
            want = to_f32(g * d * Fraction(ts))
            want = -want if c & 8 else want
            assert out[i] == want and np.signbit(out[i]) == bool(c & 8), (c, s, ts)
    # MXFP4: exact power-of-two products
    cfg = orc.Cfg(format=orc.MXFP4)
    sc = np.array([0, 1, 100, 127, 200, 250, 126, 50, 3, 129, 130, 131, 90, 110, 140, 160], dtype=np.uint8)
    out = orc.dequantize(cfg, codes, sc, 1.0, 1, 512)
    nib = _unpack(codes)
    for i in range(512):
        want = float(Fraction(float(E2M1[nib[i] & 7])) * Fraction(2) ** (int(sc[i // 32]) - 127))
        want = -want if nib[i] & 8 else want
        assert out[i] == np.float32(want)


def test_dequant_bf16_is_rne_of_fp32(orc):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, 512, dtype=np.uint8)
    sc = rng.integers(0, 0x7F, 64, dtype=np.uint8)
    cfg = orc.Cfg()
    f = orc.dequantize(cfg, codes, sc, 0.0123, 1, 1024)
    b = orc.dequantize(cfg, codes, sc, 0.0123, 1, 1024, out_bf16=True)
    assert (b == W.f32_to_bf16_rne(f)).all()


def test_dequant_bf16_ties_go_to_even(orc):
    # with d = 1, ts = 1 + 2^-8 and 1 + 3*2^-8 put the fp32 results of the power-of-two
    # codewords exactly halfway between two bf16 values; torch's fp32 -> bf16 cast
    # rounds half to even
    codes = np.arange(256, dtype=np.uint8)  # every pair of codes
    cfg = orc.Cfg()
    for ts in (1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8):  # ties below an even / an odd bf16 value
        sc = np.full(32, 0x38, dtype=np.uint8)  # d = 1
        f = orc.dequantize(cfg, codes, sc, ts, 1, 512)
        b = orc.dequantize(cfg, codes, sc, ts, 1, 512, out_bf16=True)
        want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert (b == want).all()
        assert ((f.view(np.uint32) & 0xFFFF) == 0x8000).sum() >= 64  # ties are really there


def test_special_blocks(orc):
    cfg = orc.Cfg()
    x = np.zeros((1, 96), dtype=np.float32)
    x[0, 16:32] = -0.0                       # block 1: all negative zeros
    x[0, 32] = 1000.0                        # block 2: single outlier
    x[0, 48:64] = np.float32(2.0 ** -130)    # block 3: bf16 subnormals
    x[0, 64:80] = [0, .5, 1, 1.5, 2, 3, 4, 6, -6, -4, -3, -2, -1.5, -1, -.5, -0.]  # block 4: on grid
    xh = _bf16(x)
    xh[0, 80:96] = _bf16(np.ones(16, dtype=np.float32))
    xh[0, 85] = 0x7FC0                       # block 5: NaN inside
    xh = np.concatenate([xh, _bf16(np.ones((1, 32), dtype=np.float32))], axis=1)
    xh[0, 100] = 0x7F80                      # block 6: +Inf inside
    xh[0, 127] = 0xFF80                      # block 7: -Inf inside
    codes, scales = orc.quantize(cfg, orc.RTN, xh, 1.0)
    nib = _unpack(codes)
    assert scales[6] == 0x7F and scales[7] == 0x7F and (nib[96:128] == 0).all()
    deq = orc.dequantize(cfg, codes, scales, 1.0, 1, 128)
    assert (deq.view(np.uint32)[80:] == 0x7FC00000).all()   # canonical quiet NaN for the whole block
    assert (orc.dequantize(cfg, codes, scales, 1.0, 1, 128, out_bf16=True)[80:] == 0x7FC0).all()
    assert scales[0] == 0 and (nib[:16] == 0).all()          # all-zero block: zero scale and codes
    assert scales[1] == 0 and (nib[16:32] == 8).all()        # -0 keeps its sign
    assert nib[32] == 7 and (nib[33:48] == 0).all()          # outlier at the max, rest zero
    assert (nib[48:64] == 0).all()                           # subnormals vanish at this scale
    assert scales[5] == 0x7F and (nib[80:96] == 0).all()     # non-finite block
    # on-grid block: its own scale (amax 6 -> t = 6/6 = 1 -> code 0x38) gives the exact codes
    assert scales[4] == 0x38
    assert list(nib[64:80]) == [0, 1, 2, 3, 4, 5, 6, 7, 15, 14, 13, 12, 11, 10, 9, 8]
    cfgm = orc.Cfg(format=orc.MXFP4)
    cm, sm = orc.quantize(cfgm, orc.RTN, xh, 1.0)
    assert sm[0] == 0 and sm[2] == 0xFF and sm[3] == 0xFF    # MX: zero block -> 2^-127, NaN/Inf -> 0xFF
    assert (_unpack(cm)[64:128] == 0).all()
    dm = orc.dequantize(cfgm, cm, sm, 1.0, 1, 128)
    assert (dm.view(np.uint32)[64:] == 0x7FC00000).all()


def test_guide_pack_unpack_roundtrip(orc):
    rng = np.random.default_rng(2)
    R, C = 16, 128
    codes = rng.integers(0, 256, R * C // 2, dtype=np.uint8)
    scales = rng.integers(0, 256, R * C // 16, dtype=np.uint8)
    cfg = orc.Cfg()
    bits, gs = orc.guide_pack(cfg, codes, scales, R, C)
    assert (np.unpackbits(bits, bitorder="little") == (_unpack(codes) & 1)).all()
    assert (gs == scales).all()
    mant, so = orc.guide_unpack(cfg, bits, gs, R, C)
    assert (mant == (_unpack(codes) & 1)).all() and (so == scales).all()
    bits2, _ = orc.guide_pack(cfg, _pack(mant), so, R, C)
    assert (bits2 == bits).all()


def test_cache_is_one_sixth_of_full_codes_for_deep_half():
    # 1 mantissa bit + 8-bit scale per 16 elements vs 4-bit code + scale, on 20 of 40 layers
    per_layer = W.C4_EXPERTS * W.C4_W_SHAPE[0] * W.C4_W_SHAPE[1] + W.C4_A_SHAPE[0] * W.C4_A_SHAPE[1]
    guide = W.C4_DEEP * per_layer * Fraction(1, 8) + W.C4_DEEP * per_layer * Fraction(1, 16)
    full = W.C4_LAYERS * per_layer * Fraction(1, 2) + W.C4_LAYERS * per_layer * Fraction(1, 16)
    assert guide == 314_572_800 and full == 1_887_436_800
    assert guide / full == Fraction(1, 6)


def _block_with(vals_codes):
    """16 (x value, rollout code) pairs -> bf16 row, packed rollout codes."""
    x = np.array([v for v, _ in vals_codes], dtype=np.float32)[None, :]
    r = np.array([c for _, c in vals_codes], dtype=np.uint8)
    return _bf16(x), _pack(r)


def test_guide_mismatch_counts_the_bracket_cases(orc):
    # unit scale (rollout block scale 0x38 = 1.0, tensor scale 1): v = |x|
    cases = [(2.4, 5), (2.4, 6), (2.4, 0xD), (2.0, 5), (2.0, 4), (-0.3, 9), (0.3, 8), (7.0, 6)]
    # 2.4 brackets {2, 3}: code 5 (3.0) is named by its LSB; code 6 (4.0, LSB 0) is not, the bit
    # picks 2.0 instead; -3.0 has the right magnitude but the other sign.  2.0 is a codeword:
    # it keeps code 4 whatever the bit.  7.0 clamps to the codeword 6 (code 7).
    cases += [(1.0, 2)] * 8
    xh, rc = _block_with(cases)
    nan_block, nan_rc = _block_with([(1.0, 2)] * 16)
    nan_block[0, 3] = 0x7FC0                       # non-finite input: block left out
    sb, sb_rc = _block_with([(1.0, 2)] * 16)       # its scale will be the NaN code: left out
    x = np.concatenate([xh, nan_block, sb], axis=1)
    r = np.concatenate([rc, nan_rc, sb_rc])
    scales = np.array([0x38, 0x38, 0x7F], dtype=np.uint8)
    n, nonadj, mism = orc.guide_mismatch(orc.Cfg(), x, 1.0, r, scales)
    assert (n, nonadj, mism) == (16, 3, 5)


@pytest.mark.parametrize("fmt,grid,rht", [(0, 0, False), (1, 0, False), (0, 1, True), (1, 1, False)])
def test_guide_mismatch_is_zero_for_the_own_rtn_and_recounts(orc, fmt, grid, rht):
    R, C = 48, 256
    x = W.c5_x(R, C, seed=8)
    cfg = orc.Cfg(format=fmt, grid=grid, rht16=rht, rht_seed=7)
    ts = orc.tensor_scale(cfg, x) if fmt == 0 else 1.0
    rc, rs = orc.quantize(cfg, orc.RTN, x, ts)
    assert orc.guide_mismatch(cfg, x, ts, rc, rs) == (R * C, 0, 0)
    # a rollout of 1.7 x: recount from the oracle's guided codes
    xr = _bf16(_f32(x) * np.float32(1.7))
    rc2, rs2 = orc.quantize(cfg, orc.RTN, xr, ts)
    gb = np.packbits((_unpack(rc2) & 1).astype(np.uint8), bitorder="little")
    gc, _ = orc.quantize(cfg, orc.GUIDED, x, ts, guide_bits=gb, guide_scales=rs2)
    g, r = _unpack(gc), _unpack(rc2)
    want = (R * C, int(((g & 7) != (r & 7)).sum()), int((g != r).sum()))
    assert orc.guide_mismatch(cfg, x, ts, rc2, rs2) == want
    assert want[1] > R * C // 4
