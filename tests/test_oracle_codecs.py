"""Pins for the oracle's number formats and fp32 rounding convention (CPU).

Each check compares the oracle with something other than itself: the cited
code tables, exact rational arithmetic, or torch's own fp8 conversions.
"""
import json
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import to_f32, bf16_values_nonneg_finite, bits_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_grid_matches_cited_table(orc):
    g = json.load(open(os.path.join(GOLDEN, "e2m1_grid.json")))
    assert [orc.grid_value(0, k) for k in range(8)] == g["e2m1_magnitudes"]
    assert [orc.grid_value(1, k) for k in range(8)] == g["uniform_magnitudes"]


def test_grid_dequant_of_all_16_codes_at_unit_scale(orc):
    # d = 1 is E4M3 code 0x38 (exponent field 7 = bias); s_t = 1.
    g = json.load(open(os.path.join(GOLDEN, "e2m1_grid.json")))
    cfg = orc.Cfg(format=orc.NVFP4)
    codes = np.array([(2 * j + 1) << 4 | (2 * j) for j in range(8)], dtype=np.uint8)  # codes 0..15
    out = orc.dequantize(cfg, codes, np.array([0x38], dtype=np.uint8), 1.0, 1, 16)
    mags = g["e2m1_magnitudes"]
    assert list(out[:8]) == mags
    assert list(out[8:]) == [-m for m in mags]
    assert np.signbit(out[8])  # code 8 is -0.0
    # the page's adjacent codewords 2 and 3 are neighbours in the table
    assert mags.index(3.0) == mags.index(2.0) + 1


def test_e4m3_decode_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([orc.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(t)
    assert (np.isnan(mine) == nan).all()
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert (mine[~nan] == t[~nan]).all()
    assert orc.e4m3_decode(0x7E) == 448.0 and orc.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne_below_464(orc):
    v = bf16_values_nonneg_finite()
    v = v[v < 464.0]
    rng = np.random.default_rng(5)
    extra = rng.uniform(0, 464, 20000).astype(np.float32)
    tiny = (rng.uniform(0, 2 ** -6, 5000)).astype(np.float32)
    # exact E4M3 midpoints and their fp32 neighbours
    mids = []
    for c in range(0x7E):
        a, b = orc.e4m3_decode(c), orc.e4m3_decode(c + 1)
        m = np.float32((a + b) / 2)
        mids += [m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    vals = np.concatenate([v, extra, tiny, np.array(mids, dtype=np.float32)])
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([orc.e4m3_encode(float(x)) for x in vals], dtype=np.uint8)
    assert (mine == ref).all()


def test_e4m3_encode_saturates(orc):
    for t in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38, float("inf")]:
        assert orc.e4m3_encode(t) == 0x7E
    assert orc.e4m3_encode(float("nan")) == 0x7F


def test_e8m0_decode_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    mine = np.array([orc.e8m0_decode(c) for c in range(256)])
    assert np.isnan(mine[255]) and np.isnan(t[255])
    assert (mine[:255] == t[:255]).all()


@pytest.mark.parametrize("op", ["mul", "div", "add", "sub"])
def test_fp32_rounding_helpers_are_correctly_rounded(orc, op):
    rng = random.Random(11)
    f = {"mul": orc.mul32, "div": orc.div32, "add": orc.add32, "sub": orc.sub32}[op]
    exact = {"mul": lambda a, b: a * b, "div": lambda a, b: a / b,
             "add": lambda a, b: a + b, "sub": lambda a, b: a - b}[op]
    cases = []
    for _ in range(3000):
        # mix of normal, subnormal and random bit patterns (finite, b != 0)
        a = bits_f32(rng.getrandbits(32) & 0x7F7FFFFF) * rng.choice([1, -1])
        b = bits_f32(rng.getrandbits(32) & 0x7F7FFFFF) * rng.choice([1, -1])
        cases.append((a, b))
    for _ in range(3000):
        a = float(np.float32(rng.uniform(-8, 8)))
        b = float(np.float32(rng.choice([rng.uniform(1e-40, 1e-36), rng.uniform(-4, 4), 2688.0, 3136.0])))
        cases.append((a, b))
    for a, b in cases:
        if b == 0.0:
            continue
        q = exact(Fraction(a), Fraction(b))
        want = to_f32(q)
        got = f(a, b)
        if want == 0.0:
            assert got == 0.0
        else:
            assert got == want, (op, a, b, got, want)
