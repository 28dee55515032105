"""GPU parity of the MXFP4 matrix product with the oracle.

The oracle sums the exact products in float64.  The matrix cores sum in fp32
in an order of their own, so the check is the worst-case bound of any fp32
summation of K products, each product exact (an E2M1 value has 2 significant
bits, so a product of two has at most 4 and fits fp32 whenever it is in range):
    |C - C_exact| <= (K + 1) * 2^-24 * sum_k |a b| + K * 2^-149,
the second term covering results below fp32's normal range.  bf16 output adds
the final rounding: + 2^-8 (|C_exact| + that bound).

Inputs are seeded random code and scale bytes (every code equally likely) and,
at small sizes, the oracle's own MXFP4 quantization of Gaussian activations
and weights; shapes leave ragged tiles in M and N and K tails that are not a
multiple of 128.
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
    fp4q.lib()
    return fp4q


def say(*a):
    print(*a, flush=True)


def bound(K, exact, mag, bf16):
    tol = (K + 1) * 2.0 ** -24 * mag + K * 2.0 ** -149
    if bf16:
        tol = tol + 2.0 ** -8 * (np.abs(exact) + tol)
    return tol


def run(fq, a, asc, b, bsc, M, N, K, dtype, ldc=None):
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    if ldc is None:
        out = torch.full((M, N), float("nan"), dtype=dtype, device="cuda")
    else:
        out = torch.full((M, ldc), float("nan"), dtype=dtype, device="cuda")[:, :N]
    fq.fp4_gemm_mxfp4(dev(a), dev(asc), dev(b), dev(bsc), M, N, K, out=out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def check(got, exact, mag, K, bf16, tag):
    tol = bound(K, exact, mag, bf16)
    err = np.abs(got - exact)
    bad = ~(err <= tol)
    rel = float((err / np.maximum(mag, 1e-300)).max()) if err.size else 0.0
    say(f"{tag}: max |err|/sum|ab| = {rel:.3e} (fp32 bound {(K + 1) * 2.0 ** -24:.3e})")
    if bad.any():
        where = np.argwhere(bad)
        say(f"{tag}: bad rows {np.unique(where[:, 0])[:20]} cols {np.unique(where[:, 1])[:40]}")
    assert not bad.any(), f"{tag}: {int(bad.sum())} results outside the bound, first at {np.argwhere(bad)[0]}"


SHAPES = [(128, 128, 128), (1, 1, 32), (200, 136, 96), (257, 129, 160), (384, 256, 1024), (130, 300, 4096),
          (64, 520, 224)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_random_operands(fq, M, N, K, dtype):
    say(f"gemm random M={M} N={N} K={K} {dtype}")
    a, asc = W.mx_operand(M, K, seed=M, stream=0)
    b, bsc = W.mx_operand(N, K, seed=N, stream=2)
    exact, mag = O.gemm_mx(a, asc, b, bsc, M, N, K)
    got = run(fq, a, asc, b, bsc, M, N, K, dtype)
    check(got, exact, mag, K, dtype == torch.bfloat16, f"random {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,ldc", [(150, 70, 256, 96), (130, 300, 1024, 320), (300, 200, 512, 232)])
def test_padded_output_rows(fq, M, N, K, ldc):
    # columns N .. ldc - 1 of every row must keep their sentinel: a store past N would land there
    say(f"gemm padded ldc M={M} N={N} K={K} ldc={ldc}")
    a, asc = W.mx_operand(M, K, seed=5, stream=0)
    b, bsc = W.mx_operand(N, K, seed=6, stream=0)
    exact, mag = O.gemm_mx(a, asc, b, bsc, M, N, K)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    buf = torch.full((M, ldc), -7.0, dtype=torch.float32, device="cuda")
    fq.fp4_gemm_mxfp4(dev(a), dev(asc), dev(b), dev(bsc), M, N, K, out=buf[:, :N])
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    check(h[:, :N].astype(np.float64), exact, mag, K, False, "padded")
    assert (h[:, N:] == -7.0).all(), "the product wrote past N in a padded row"


def test_quantized_gaussian_operands(fq):
    # activations N(0,1) and an expert weight N(0, 0.02^2), both quantized to MXFP4 by the oracle
    M, N, K = 256, 192, 512
    say(f"gemm quantized gaussian M={M} N={N} K={K}")
    cfg = O.Cfg(format=O.MXFP4)
    xa = W.f32_to_bf16_rne(W.normal_outliers_f32(M, K, 11, 0, 0.0, 1.0))
    xb = W.f32_to_bf16_rne(W.normal_outliers_f32(N, K, 11, 1, 0.0, 1.0, sigma=0.02))
    a, asc = O.quantize(cfg, O.RTN, xa)
    b, bsc = O.quantize(cfg, O.RTN, xb)
    exact, mag = O.gemm_mx(a, asc, b, bsc, M, N, K)
    for dtype in (torch.float32, torch.bfloat16):
        got = run(fq, a, asc, b, bsc, M, N, K, dtype)
        check(got, exact, mag, K, dtype == torch.bfloat16, f"quantized gaussian {dtype}")


def test_extreme_scales(fq):
    # scales near both ends of E8M0: products far below fp32's normal range (flushed or subnormal)
    # and products near its top
    M, N, K = 128, 128, 256
    for lo, hi, tag in [(1, 12, "tiny"), (60, 70, "small"), (175, 183, "large")]:
        say(f"gemm extreme scales {tag}")
        a, asc = W.mx_operand(M, K, seed=lo, stream=0, scale_lo=lo, scale_hi=hi)
        b, bsc = W.mx_operand(N, K, seed=hi, stream=0, scale_lo=lo, scale_hi=hi)
        exact, mag = O.gemm_mx(a, asc, b, bsc, M, N, K)
        if tag == "large":
            assert np.isfinite(exact).all() and mag.max() < 3e38
        got = run(fq, a, asc, b, bsc, M, N, K, torch.float32)
        check(got, exact, mag, K, False, f"scales {tag}")


def test_nan_scale_blocks(fq):
    M, N, K = 130, 140, 256
    say("gemm NaN scale blocks")
    a, asc = W.mx_operand(M, K, seed=21, stream=0)
    b, bsc = W.mx_operand(N, K, seed=22, stream=0)
    a = a | 0x11   # no zero codes: a NaN block cannot be hidden by 0 * NaN
    b = b | 0x11
    asc = asc.copy(); bsc = bsc.copy()
    asc[3, 2] = 0xFF
    asc[129, 0] = 0xFF
    bsc[77, 7] = 0xFF
    exact, mag = O.gemm_mx(a, asc, b, bsc, M, N, K)
    got = run(fq, a, asc, b, bsc, M, N, K, torch.float32)
    nan = np.isnan(exact)
    assert nan[3].all() and nan[129].all() and nan[:, 77].all()
    assert (np.isnan(got) == nan).all(), "NaN results differ from the oracle's"
    check(np.where(nan, 0, got), np.where(nan, 0, exact), np.where(nan, 0, mag), K, False, "finite part")


def test_k_zero_writes_zeros(fq):
    out = torch.full((40, 24), 5.0, dtype=torch.float32, device="cuda")
    e = torch.empty(16, dtype=torch.uint8, device="cuda")
    fq.fp4_gemm_mxfp4(e, e, e, e, 40, 24, 0, out=out)
    torch.cuda.synchronize()
    assert (out == 0).all()


def test_empty_is_noop(fq):
    e = torch.empty(16, dtype=torch.uint8, device="cuda")
    out = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    fq.fp4_gemm_mxfp4(e, e, e, e, 0, 8, 64, out=out)
    torch.cuda.synchronize()


def test_large_tiles_ragged_sampled(fq):
    # enough 256 x 192 tiles to fill the chip, with ragged last tiles in both M and N; the output
    # rows are padded with a sentinel that no store may touch
    M, N, K = 4100, 3000, 512
    say(f"gemm large tiles ragged M={M} N={N} K={K}")
    a, asc = W.mx_operand(M, K, seed=51, stream=0)
    b, bsc = W.mx_operand(N, K, seed=52, stream=0)
    rng = np.random.default_rng(10)
    rows = np.unique(np.concatenate([rng.choice(M, 32, replace=False), np.arange(M - 8, M), np.arange(0, 4)]))
    cols = np.unique(np.concatenate([rng.choice(N, 32, replace=False), np.arange(N - 8, N), np.arange(0, 4)]))
    e_rows, m_rows = O.gemm_mx(a[rows], asc[rows], b, bsc, len(rows), N, K)
    e_cols, m_cols = O.gemm_mx(a, asc, b[cols], bsc[cols], M, len(cols), K)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    for dtype in (torch.float32, torch.bfloat16):
        buf = torch.full((M, N + 40), -7.0, dtype=dtype, device="cuda")
        fq.fp4_gemm_mxfp4(dev(a), dev(asc), dev(b), dev(bsc), M, N, K, out=buf[:, :N])
        torch.cuda.synchronize()
        h = buf.float().cpu().numpy()
        assert (h[:, N:] == -7.0).all(), "the product wrote past N in a padded row"
        got = h[:, :N].astype(np.float64)
        bf = dtype == torch.bfloat16
        check(got[rows], e_rows, m_rows, K, bf, f"large tiles rows {dtype}")
        check(got[:, cols], e_cols, m_cols, K, bf, f"large tiles cols {dtype}")


@pytest.mark.parametrize("pad", [40, 3])
def test_256x256_tiles_ragged_sampled(fq, pad):
    # 4000 x 4000 makes 256 tiles of 256 x 256 (one round) against 336 of 256 x 192 (two), so the
    # 256 x 256 configuration runs, with ragged last tiles in M and N.  Rows padded by 40 elements
    # keep every row 16-byte aligned (whole tiles go through LDS); a padding of 3 does not (every
    # tile stores element by element).  The padding holds a sentinel no store may touch.
    M, N, K = 4000, 4000, 512
    say(f"gemm 256x256 tiles M={M} N={N} K={K} pad={pad}")
    a, asc = W.mx_operand(M, K, seed=61, stream=0)
    b, bsc = W.mx_operand(N, K, seed=62, stream=0)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), np.arange(M - 8, M), np.arange(0, 4),
                                     np.arange(3840, 3844)]))
    cols = np.unique(np.concatenate([rng.choice(N, 24, replace=False), np.arange(N - 8, N), np.arange(0, 4),
                                     np.arange(3840, 3844)]))
    e_rows, m_rows = O.gemm_mx(a[rows], asc[rows], b, bsc, len(rows), N, K)
    e_cols, m_cols = O.gemm_mx(a, asc, b[cols], bsc[cols], M, len(cols), K)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    for dtype in (torch.float32, torch.bfloat16):
        buf = torch.full((M, N + pad), -7.0, dtype=dtype, device="cuda")
        fq.fp4_gemm_mxfp4(dev(a), dev(asc), dev(b), dev(bsc), M, N, K, out=buf[:, :N])
        torch.cuda.synchronize()
        h = buf.float().cpu().numpy()
        assert (h[:, N:] == -7.0).all(), "the product wrote past N in a padded row"
        got = h[:, :N].astype(np.float64)
        bf = dtype == torch.bfloat16
        check(got[rows], e_rows, m_rows, K, bf, f"256x256 rows {dtype}")
        check(got[:, cols], e_cols, m_cols, K, bf, f"256x256 cols {dtype}")


def test_square_16384_sampled(fq):
    # the square product bench.py times (256 x 256 tiles, 16 rounds): 8 sampled rows x all columns and
    # all rows x 8 sampled columns, bf16 out
    M = N = K = 16384
    say(f"gemm square M={M} N={N} K={K}")
    a, asc = W.mx_operand(M, K, seed=71, stream=0)
    b, bsc = W.mx_operand(N, K, seed=72, stream=0)
    rng = np.random.default_rng(13)
    rows = np.sort(np.concatenate([rng.choice(M - 2, 6, replace=False), [M - 2, M - 1]]))
    cols = np.sort(np.concatenate([rng.choice(N - 2, 6, replace=False), [N - 2, N - 1]]))
    e_rows, m_rows = O.gemm_mx(a[rows], asc[rows], b, bsc, len(rows), N, K)
    e_cols, m_cols = O.gemm_mx(a, asc, b[cols], bsc[cols], M, len(cols), K)
    got = run(fq, a, asc, b, bsc, M, N, K, torch.bfloat16)
    check(got[rows], e_rows, m_rows, K, True, "square rows")
    check(got[:, cols], e_cols, m_cols, K, True, "square cols")


def test_full_size_expert_gemm_sampled(fq):
    # the benchmark's product: activations [8192, 4096] x expert weight [1536, 4096]^T, bf16 and fp32 out;
    # 64 sampled rows x all columns and all rows x 48 sampled columns checked against the oracle
    M, N, K = W.GEMM_SHAPE
    say(f"gemm full size M={M} N={N} K={K}")
    a, asc = W.mx_operand(M, K, seed=41, stream=0)
    b, bsc = W.mx_operand(N, K, seed=42, stream=0)
    rng = np.random.default_rng(9)
    rows = np.sort(rng.choice(M, 64, replace=False))
    cols = np.sort(rng.choice(N, 48, replace=False))
    e_rows, m_rows = O.gemm_mx(a[rows], asc[rows], b, bsc, len(rows), N, K)
    e_cols, m_cols = O.gemm_mx(a, asc, b[cols], bsc[cols], M, len(cols), K)
    for dtype in (torch.bfloat16, torch.float32):
        got = run(fq, a, asc, b, bsc, M, N, K, dtype)
        bf = dtype == torch.bfloat16
        check(got[rows], e_rows, m_rows, K, bf, f"full size rows {dtype}")
        check(got[:, cols], e_cols, m_cols, K, bf, f"full size cols {dtype}")


@pytest.mark.parametrize("K", [512, 160])
def test_grouped_experts_vs_oracle(fq, K):
    # eight experts with their own token counts (one empty) and weights: K = 512 runs as one launch,
    # K = 160 as one launch per product
    Ms = [300, 0, 129, 700, 64, 1, 256, 413]
    N = 192
    say(f"gemm grouped K={K} Ms={Ms}")
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    prods, refs = [], []
    for e, M in enumerate(Ms):
        a, asc = W.mx_operand(M, K, seed=70 + e, stream=0)
        b, bsc = W.mx_operand(N, K, seed=90 + e, stream=0)
        prods.append((dev(a), dev(asc), dev(b), dev(bsc), M, N, K))
        refs.append(O.gemm_mx(a, asc, b, bsc, M, N, K) if M else None)
    for dtype in (torch.float32, torch.bfloat16):
        outs = fq.fp4_gemm_mxfp4_grouped(prods, dtype=dtype)
        torch.cuda.synchronize()
        for e, (M, out, ref) in enumerate(zip(Ms, outs, refs)):
            if M:
                check(out.float().cpu().numpy().astype(np.float64), ref[0], ref[1], K, dtype == torch.bfloat16,
                      f"grouped expert {e} {dtype}")


@pytest.mark.parametrize("K,dtype", [(512, torch.float32), (4096, torch.bfloat16)])
def test_grouped_large_tiles_sampled(fq, K, dtype):
    # 8 experts x 1024 tokens x [1536, K] weights: 256 tiles of 256 x 192 in one launch; K = 4096 with
    # bf16 out is the grouped product bench.py times (16 stages, so the K loop body runs)
    E, M, N = 8, 1024, 1536
    say(f"gemm grouped large E={E} M={M} N={N} K={K} {dtype}")
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x).ravel()).cuda()
    rng = np.random.default_rng(12)
    prods, host = [], []
    for e in range(E):
        a, asc = W.mx_operand(M, K, seed=110 + e, stream=0)
        b, bsc = W.mx_operand(N, K, seed=130 + e, stream=0)
        prods.append((dev(a), dev(asc), dev(b), dev(bsc), M, N, K))
        host.append((a, asc, b, bsc))
    outs = fq.fp4_gemm_mxfp4_grouped(prods, dtype=dtype)
    torch.cuda.synchronize()
    for e, (a, asc, b, bsc) in enumerate(host):
        rows = np.sort(np.concatenate([[0, M - 1], rng.choice(np.arange(1, M - 1), 14, replace=False)]))
        ref, mag = O.gemm_mx(a[rows], asc[rows], b, bsc, len(rows), N, K)
        got = outs[e].float().cpu().numpy()[rows].astype(np.float64)
        check(got, ref, mag, K, dtype == torch.bfloat16, f"grouped large expert {e} K={K}")
