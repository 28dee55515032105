"""Pins for the oracle's per-element encode (RTN / SR / guided), CPU.

Brute force and closed forms computed here with exact rationals:
* RTN: argmin over the 8 grid values, ties to the even code.
* SR: the number of the 256 random bytes u that round up equals
  round-half-down(256 f), f the position of the value inside its bracket.
* guided: the result is one of the two bracketing codewords, and its LSB is
  the guide bit whenever the value is not on a codeword.
Exhaustive over every finite non-negative bf16 value, plus fp32 values
around every grid point and midpoint.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from exact import bf16_values_nonneg_finite, grid_values, bracket

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _near_points(grid):
    G = grid_values(grid)
    pts = set(G) | {(G[k] + G[k + 1]) / 2 for k in range(7)} | {G[-1] + 1, G[-1] + Fraction(1, 2)}
    out = []
    for p in sorted(pts):
        c = np.float32(float(p))
        u = np.array([c], dtype=np.float32).view(np.uint32)[0]
        for d in range(-64, 65):
            w = int(u) + d
            if w >= 0:
                out.append(np.array([w], dtype=np.uint32).view(np.float32)[0])
    return np.array(out, dtype=np.float32)


def _values(grid):
    v = np.concatenate([bf16_values_nonneg_finite(), _near_points(grid)])
    rng = np.random.default_rng(3)
    v = np.concatenate([v, rng.uniform(0, 9, 20000).astype(np.float32)])
    return v


@pytest.mark.parametrize("grid", [0, 1])
def test_rtn_is_nearest_with_ties_to_even(orc, grid):
    G = np.array([float(g) for g in grid_values(grid)])
    v = _values(grid)
    got = orc.encode_many(grid, orc.RTN, v)
    vc = np.minimum(v.astype(np.float64), G[-1])
    d = np.abs(vc[:, None] - G[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8) % 2 == 0)[None, :]
    want = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    assert (got == want).all()
    # error bound: within half a grid step of the clamped value
    gap = np.diff(G)
    k = got.astype(int)
    lo_gap = np.where(k > 0, gap[np.maximum(k - 1, 0)], gap[0])
    hi_gap = np.where(k < 7, gap[np.minimum(k, 6)], gap[-1])
    err = np.abs(G[k] - vc)
    assert (err <= np.maximum(lo_gap, hi_gap) / 2).all()


@pytest.mark.parametrize("grid", [0, 1])
def test_sr_up_count_is_round_half_down_of_256f(orc, grid):
    v = bf16_values_nonneg_finite()
    G = grid_values(grid)
    n = v.size
    vv = np.repeat(v, 256)
    uu = np.tile(np.arange(256, dtype=np.uint32), n)
    got = orc.encode_many(grid, orc.SR, vv, uu).reshape(n, 256).astype(int)
    for i in range(0, n, 7):  # exact rational check on a stride of all values
        x = Fraction(float(v[i]))
        klo, khi, vc = bracket(grid, x)
        row = got[i]
        assert set(np.unique(row)) <= {klo, khi}
        if klo == khi:
            assert (row == klo).all()
            continue
        f = (vc - G[klo]) / (G[khi] - G[klo])
        t = 256 * f
        want_up = math.ceil(t - Fraction(1, 2))  # round half down
        assert int((row == khi).sum()) == want_up
        # up decisions are the lowest bytes u: u < want_up
        assert (row[:want_up] == khi).all() and (row[want_up:] == klo).all()


def test_sr_bias_bound(orc):
    # |E[q] - v| <= gap/512 for every bf16 value (8 random bits per element)
    v = bf16_values_nonneg_finite()[::5]
    v = v[v <= 6]
    n = v.size
    got = orc.encode_many(0, orc.SR, np.repeat(v, 256), np.tile(np.arange(256, dtype=np.uint32), n))
    G = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mean = G[got.reshape(n, 256)].mean(axis=1)
    k = np.searchsorted(G, v, side="right") - 1
    gap = np.where(k < 7, np.diff(np.append(G, 8.0))[np.minimum(k, 7)], 2.0)
    assert (np.abs(mean - v.astype(np.float64)) <= gap / 512 + 1e-12).all()


@pytest.mark.parametrize("grid", [0, 1])
def test_guided_picks_the_bracket_member_with_the_guide_lsb(orc, grid):
    v = _values(grid)
    G = grid_values(grid)
    for b in (0, 1):
        got = orc.encode_many(grid, orc.GUIDED, v, np.full(v.size, b, dtype=np.uint32)).astype(int)
        Gf = np.array([float(g) for g in G])
        vc = np.minimum(v.astype(np.float64), Gf[-1])
        klo = np.searchsorted(Gf, vc, side="right") - 1
        khi = np.searchsorted(Gf, vc, side="left")
        assert ((got == klo) | (got == khi)).all()
        off = klo != khi
        assert ((got[off] & 1) == b).all()
        assert (got[~off] == klo[~off]).all()


def test_guided_with_own_rtn_bit_equals_rtn(orc):
    for grid in (0, 1):
        v = _values(grid)
        rtn = orc.encode_many(grid, orc.RTN, v)
        guided = orc.encode_many(grid, orc.GUIDED, v, (rtn & 1).astype(np.uint32))
        assert (guided == rtn).all()


def test_adjacent_codewords_differ_in_lsb():
    # the 1-bit guide can only name a bracket member because neighbours alternate LSB
    for k in range(7):
        assert (k & 1) != ((k + 1) & 1)


def test_worked_example(orc):
    ex = json.load(open(os.path.join(GOLDEN, "trace_worked_example.json")))
    for c in ex["rtn"]:
        k = orc.encode(0, orc.RTN, c["v"])
        assert k == c["code"] and orc.grid_value(0, k) == c["value"]
    for c in ex["guided"]:
        k = orc.encode(0, orc.GUIDED, c["v"], c["rollout_code"] & 1)
        assert k == c["code"] and orc.grid_value(0, k) == c["value"]
        assert (k & 1) == c["guide_bit"]


def test_breakpoints_of_rtn_are_the_midpoints(orc):
    # scan fp32 patterns in [0.125, 8): RTN changes exactly at the midpoints
    lo = np.array([0.125], dtype=np.float32).view(np.uint32)[0]
    hi = np.array([8.0], dtype=np.float32).view(np.uint32)[0]
    bp, n = orc.encode_breakpoints(0, orc.RTN, 0, int(lo), int(hi))
    vals = bp.view(np.float32)
    # tie to even: 0.25->0 (up just above), 0.75->2 (at), 1.25->2, 1.75->4 (at), 2.5->4, 3.5->6 (at), 5->6
    expect_at = {0.75, 1.75, 3.5}
    expect_above = {0.25, 1.25, 2.5, 5.0}
    assert n == 7
    for m, val in zip([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], vals):
        if m in expect_at:
            assert val == np.float32(m)
        else:
            assert val == np.nextafter(np.float32(m), np.float32(9))
    assert expect_at | expect_above == {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0}
