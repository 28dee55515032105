"""Pins for the oracle's Philox4x32-10 and 16-point RHT (CPU).

Philox: cross-checked against rocRAND's Philox4x32-10 engine (a library
routine, compiled here as host code), plus byte-histogram statistics.
RHT16: closed form of the Sylvester Hadamard matrix, the O(n^2) product where
every partial sum is exact, involution, basis vectors and norm preservation.
The butterfly's rounding order beyond exact cases is a reading (parity
unpinned there).
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _hadamard16():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    d = tempfile.mkdtemp()
    exe = os.path.join(d, "philox_ref")
    subprocess.run([hipcc, "-O1",
                    os.path.join(HERE, "rocrand_philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(cases):
        inp = "\n".join(" ".join(str(v) for v in c) for c in cases) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(t) for t in line.split()) for line in out.strip().splitlines()]
    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand(orc, rocrand_ref):
    rng = np.random.default_rng(1)
    cases = [(0, 0, 0, 0, 0, 0), (0, 0, 1, 0, 7, 0), (5, 0, 0, 0, 1, 0), (12345, 0, 0, 0, 0xFFFFFFFF, 7)]
    for _ in range(300):
        c = rng.integers(0, 2 ** 32, 4, dtype=np.uint64)
        k = rng.integers(0, 2 ** 32, 2, dtype=np.uint64)
        cases.append((int(c[0]), int(c[1]) & 0x3FFFFFFF, int(c[2]), int(c[3]), int(k[0]), int(k[1])))
    ref = rocrand_ref(cases)
    assert len(ref) == len(cases)
    for c, r in zip(cases, ref):
        assert orc.philox4x32_10(c[:4], c[4:]) == r, c


def test_philox_byte_histogram(orc):
    counts = np.zeros(256, dtype=np.int64)
    for g in range(4096):
        w = orc.philox4x32_10((g, 0, 0, 0), (1, 0))
        b = np.frombuffer(np.array(w, dtype=np.uint32).tobytes(), dtype=np.uint8)
        np.add.at(counts, b, 1)
    n = counts.sum()
    exp = n / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 255 + 6 * np.sqrt(2 * 255)  # ~6 sigma of a chi2(255)


def test_rht_signs_definition(orc):
    for seed in (0, 1, 7, 2 ** 40 + 3):
        w = orc.philox4x32_10((0, 0, 1, 0), (seed & 0xFFFFFFFF, seed >> 32))
        assert orc.rht_signs(seed) == (w[0] & 0xFFFF)


@pytest.mark.parametrize("seed", [7, 0, 123456789])
def test_rht_basis_vectors_are_scaled_hadamard_columns(orc, seed):
    H = _hadamard16()
    s = orc.rht_signs(seed)
    D = np.array([-1 if (s >> j) & 1 else 1 for j in range(16)])
    for k in range(16):
        e = np.zeros(16, dtype=np.float32)
        e[k] = 1.0
        y = orc.rht16_vec(e, s)
        assert (y.astype(np.float64) == 0.25 * D[k] * H[:, k]).all()


@pytest.mark.parametrize("seed", [7, 99])
def test_rht_equals_exact_product_on_small_integers(orc, seed):
    H = _hadamard16()
    s = orc.rht_signs(seed)
    D = np.array([-1 if (s >> j) & 1 else 1 for j in range(16)])
    rng = np.random.default_rng(seed)
    for _ in range(500):
        x = rng.integers(-1000, 1001, 16)
        y = orc.rht16_vec(x.astype(np.float32), s)
        exact = (H @ (D * x)) / 4.0  # all partial sums are small integers: exact in fp32
        assert (y.astype(np.float64) == exact).all()
        back = orc.rht16_vec(y, s, inverse=True)
        assert (back.astype(np.float64) == x).all()


def test_rht_preserves_norm(orc):
    s = orc.rht_signs(7)
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = rng.standard_normal(16).astype(np.float32)
        y = orc.rht16_vec(x, s)
        assert abs(np.linalg.norm(y.astype(np.float64)) - np.linalg.norm(x.astype(np.float64))) < 1e-5 * np.linalg.norm(x)
        H = _hadamard16()
        D = np.array([-1 if (s >> j) & 1 else 1 for j in range(16)])
        assert np.allclose(y, (H @ (D * x.astype(np.float64))) / 4.0, rtol=0, atol=1e-5)


def test_rht_matrix_form_matches_vector_form(orc):
    s = orc.rht_signs(7)
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((4, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = orc.rht16(x, 7).reshape(4, 64)
    for r in range(4):
        for c in range(0, 64, 16):
            xv = (x[r, c:c + 16].astype(np.uint32) << 16).view(np.float32)
            assert (orc.rht16_vec(xv, s) == y[r, c:c + 16]).all()
