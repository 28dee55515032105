"""Pins for the oracle's MXFP4 matrix product (CPU).

The product is C = A * B^T with A [M, K] and B [N, K] given as MXFP4 codes
and E8M0 scales along K [TETRAJET section 3: per-group scales; section 4: the
matrix products of every linear layer take MXFP4 operands].  Each check
compares orc_gemm_mx with something other than itself: closed forms over the
cited E2M1 table, the separately pinned dequantization followed by numpy's
matmul, and exact invariants (transposition, sign, power-of-two scaling).
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = json.load(open(os.path.join(GOLDEN, "e2m1_grid.json")))["e2m1_magnitudes"]


def _pack(codes):
    """uint8 codes 0..15 (one per element, row-major) -> packed nibbles, element i in nibble i%2 of byte i/2."""
    c = np.asarray(codes, dtype=np.uint8).ravel()
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def _random(rng, rows, K, lo=110, hi=145):
    codes = rng.integers(0, 256, rows * K // 2, dtype=np.uint8)
    scales = rng.integers(lo, hi, rows * K // 32, dtype=np.uint8)
    return codes, scales


@pytest.mark.parametrize("ca,ea,cb,eb,K", [(7, 126, 3, 129, 32), (2, 127, 2, 127, 64), (9, 100, 15, 160, 96),
                                           (1, 131, 12, 120, 128), (0, 140, 7, 127, 32)])
def test_constant_operands_closed_form(orc, ca, ea, cb, eb, K):
    # every element of A is code ca at scale 2^(ea-127), every element of B code cb at 2^(eb-127):
    # C = K * (+-G[ca]) * (+-G[cb]) * 2^(ea + eb - 254)
    M, N = 3, 2
    a = _pack(np.full(M * K, ca)); b = _pack(np.full(N * K, cb))
    asc = np.full(M * K // 32, ea, np.uint8); bsc = np.full(N * K // 32, eb, np.uint8)
    c, mag = orc.gemm_mx(a, asc, b, bsc, M, N, K)
    va = (-1 if ca & 8 else 1) * E2M1[ca & 7] * 2.0 ** (ea - 127)
    vb = (-1 if cb & 8 else 1) * E2M1[cb & 7] * 2.0 ** (eb - 127)
    assert (c == K * va * vb).all()
    assert (mag == K * abs(va * vb)).all()


def test_worked_example_two_blocks(orc):
    # K = 64: A's first block is 6.0 at scale 1/2 (values 3), its second 1.0 at scale 8 (values 8);
    # B's first block holds 1.5 then -0.5 (16 each) at scale 4 (values 6, -2), its second -2 at scale 1/4
    # (values -0.5).  C = 16*3*6 + 16*3*(-2) + 32*8*(-0.5) = 288 - 96 - 128 = 64.
    a = _pack([7] * 32 + [2] * 32)
    b = _pack([3] * 16 + [9] * 16 + [12] * 32)
    c, mag = orc.gemm_mx(a, np.array([126, 130], np.uint8), b, np.array([129, 125], np.uint8), 1, 1, 64)
    assert c[0, 0] == 64.0
    assert mag[0, 0] == 288 + 96 + 128


@pytest.mark.parametrize("k0", [0, 1, 30, 31, 32, 33, 62, 63])
def test_one_hot_row_picks_one_element(orc, k0):
    # A row 0 is zero except element k0 (code 5 = 3.0): C[0, n] = 3 * 2^(e - 127) * b(n, k0), with the
    # per-block scales of A distinct so a wrong block index changes the value.
    rng = np.random.default_rng(k0)
    M, N, K = 2, 5, 64
    codes = np.zeros(M * K, np.uint8)
    codes[k0] = 5
    codes[K:] = rng.integers(0, 16, K)
    asc = np.array([124, 131, 127, 127], np.uint8)
    bc, bsc = _random(rng, N, K)
    c, _ = orc.gemm_mx(_pack(codes), asc, bc, bsc, M, N, K)
    bv = orc.dequantize(orc.Cfg(format=orc.MXFP4), bc, bsc, 1.0, N, K).reshape(N, K).astype(np.float64)
    assert (c[0] == 3.0 * 2.0 ** (int(asc[k0 // 32]) - 127) * bv[:, k0]).all()


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (7, 5, 96), (16, 33, 256), (40, 24, 1024)])
def test_matches_dequantize_then_matmul(orc, M, N, K):
    # dequantization is pinned on its own; with scales well inside fp32's range its values are exact,
    # so numpy's float64 matmul of them gives C up to float64 summation order
    rng = np.random.default_rng(M * 1000 + N + K)
    ac, asc = _random(rng, M, K)
    bc, bsc = _random(rng, N, K)
    c, mag = orc.gemm_mx(ac, asc, bc, bsc, M, N, K)
    cfg = orc.Cfg(format=orc.MXFP4)
    A = orc.dequantize(cfg, ac, asc, 1.0, M, K).reshape(M, K).astype(np.float64)
    B = orc.dequantize(cfg, bc, bsc, 1.0, N, K).reshape(N, K).astype(np.float64)
    assert np.abs(c - A @ B.T).max() <= 1e-14 * mag.max()
    assert np.abs(mag - np.abs(A) @ np.abs(B).T).max() <= 1e-14 * mag.max()


def test_transpose_sign_and_scaling_invariants(orc):
    rng = np.random.default_rng(11)
    M, N, K = 9, 6, 160
    ac, asc = _random(rng, M, K)
    bc, bsc = _random(rng, N, K)
    c, mag = orc.gemm_mx(ac, asc, bc, bsc, M, N, K)
    # B * A^T = (A * B^T)^T: the same products in the same order
    ct, _ = orc.gemm_mx(bc, bsc, ac, asc, N, M, K)
    assert (ct == c.T).all()
    # flipping every sign bit of A negates C
    cn, magn = orc.gemm_mx(ac ^ 0x88, asc, bc, bsc, M, N, K)
    assert (cn == -c).all() and (magn == mag).all()
    # raising every scale of A by 3 multiplies C by 8 exactly
    c8, _ = orc.gemm_mx(ac, asc + 3, bc, bsc, M, N, K)
    assert (c8 == 8 * c).all()
    # clearing every sign bit makes C equal to sum |a b|
    cp, magp = orc.gemm_mx(ac & 0x77, asc, bc & 0x77, bsc, M, N, K)
    assert (cp == magp).all() and (magp == mag).all()
    assert (np.abs(c) <= mag).all()


def test_nan_scale_poisons_its_row_only(orc):
    rng = np.random.default_rng(3)
    M, N, K = 4, 3, 96
    ac, asc = _random(rng, M, K)
    bc, bsc = _random(rng, N, K)
    ac[: M * K // 2] |= 0x11   # no zero codes, so NaN * 0 cannot hide
    bc[: N * K // 2] |= 0x11
    c, _ = orc.gemm_mx(ac, asc, bc, bsc, M, N, K)
    asc2 = asc.copy()
    asc2[2 * (K // 32) + 1] = 0xFF     # row 2, block 1
    c2, _ = orc.gemm_mx(ac, asc2, bc, bsc, M, N, K)
    assert np.isnan(c2[2]).all()
    keep = [0, 1, 3]
    assert (c2[keep] == c[keep]).all()


def test_rejects_k_not_multiple_of_32(orc):
    with pytest.raises(ValueError):
        orc.gemm_mx(np.zeros(16, np.uint8), np.zeros(1, np.uint8), np.zeros(16, np.uint8),
                    np.zeros(1, np.uint8), 1, 1, 16)
