"""Seeded synthetic inputs shaped like the tensors the FP4 path quantizes.

This module holds input generation only (random draws and the fp32 -> bf16
storage rounding of the drawn values); it contains none of the quantizer's
arithmetic.  Both the HIP path (tests, bench) and the CPU oracle (tests,
CPU baseline) take their inputs from here.

Every tensor is produced in row chunks, each chunk from its own
``numpy.random.Generator(PCG64)`` stream keyed by (seed, stream, chunk), so any
row range can be regenerated on its own and the full tensor never has to be
materialised twice.  bf16 tensors are returned as ``uint16`` bit patterns.

Workloads (shapes of the MoE rollout/trainer tensors the pages talk about; the
pages name no dataset for this path, so all values are synthetic):

* ``c1``  activation 4096 x 2048, N(0,1) with 0.1 % outliers x50; the rollout
  copy adds N(0, 1e-3^2) noise (NVFP4, RTN and guided).
* ``c2``  MoE expert activations 16384 x 4096, Student-t(4); the trained copy
  is the RNE bf16 rounding of the fp32 draw, the rollout copy its truncation
  (MXFP4, RTN / SR / guided).
* ``c3``  KV cache, K and V each (131072*8) x 128, N(0,1) times a per-(head,
  dim) channel magnitude log-uniform in [0.1, 10] (NVFP4 along head_dim).
* ``c4``  guidance-cache layer: 8 expert weight slices 4096 x 1536 N(0, 0.02^2)
  and activations 8192 x 4096 N(0,1); rollout copies add relative 1e-3 noise.
* ``c5``  GEMM operand 65536 x 8192, N(0,1) with 0.5 % outliers x30 (uniform
  grid, RHT16, SR).
* ``mx_operand``  raw MXFP4 operands for the matrix product: uniformly random
  code bytes and E8M0 scale bytes drawn from a stated range (the product's
  parity inputs; the benchmark quantizes the c4 tensors instead).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

CHUNK_ROWS = 256


def f32_to_bf16_rne(a: np.ndarray) -> np.ndarray:
    """Storage rounding of drawn fp32 values to bf16 (round to nearest even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_to_bf16_rtz(a: np.ndarray) -> np.ndarray:
    """Storage truncation of drawn fp32 values to bf16 (round toward zero)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([seed, stream, chunk]))


def _chunks(rows: int, r0: int, r1: int):
    c = r0 // CHUNK_ROWS
    while c * CHUNK_ROWS < r1:
        lo = max(c * CHUNK_ROWS, r0)
        hi = min((c + 1) * CHUNK_ROWS, r1, rows)
        yield c, lo, hi
        c += 1


def _gen(rows: int, cols: int, r0: int, r1: int, fn) -> np.ndarray:
    """Assemble rows [r0, r1) from per-chunk draws fn(chunk, nrows_in_chunk) -> (n, cols)."""
    out = []
    for c, lo, hi in _chunks(rows, r0, r1):
        nrow = min((c + 1) * CHUNK_ROWS, rows) - c * CHUNK_ROWS
        blk = fn(c, nrow)
        out.append(blk[lo - c * CHUNK_ROWS: hi - c * CHUNK_ROWS])
    return np.concatenate(out, axis=0) if out else np.empty((0, cols), dtype=np.float32)


# ---------------------------------------------------------------- draws
def normal_outliers_f32(rows, cols, seed, stream, p_out, mult, r0=0, r1=None, sigma=1.0):
    r1 = rows if r1 is None else r1

    def fn(c, n):
        g = _rng(seed, stream, c)
        x = g.standard_normal((n, cols), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        if p_out > 0:
            m = g.random((n, cols), dtype=np.float32) < np.float32(p_out)
            x[m] *= np.float32(mult)
        return x
    return _gen(rows, cols, r0, r1, fn)


def noise_f32(rows, cols, seed, stream, sigma, r0=0, r1=None):
    r1 = rows if r1 is None else r1

    def fn(c, n):
        g = _rng(seed, stream, c)
        return g.standard_normal((n, cols), dtype=np.float32) * np.float32(sigma)
    return _gen(rows, cols, r0, r1, fn)


def student_t_f32(rows, cols, seed, stream, nu, r0=0, r1=None):
    r1 = rows if r1 is None else r1

    def fn(c, n):
        g = _rng(seed, stream, c)
        return g.standard_t(nu, size=(n, cols)).astype(np.float32)
    return _gen(rows, cols, r0, r1, fn)


# ---------------------------------------------------------------- workloads
@dataclass
class Workload:
    """A named tensor family; ``make(r0, r1)`` returns rows [r0, r1)."""
    name: str
    rows: int
    cols: int
    desc: str
    extra: dict = field(default_factory=dict)

    @property
    def elements(self) -> int:
        return self.rows * self.cols


# C1: NVFP4 activation with a perturbed rollout copy
def c1_shape(small: bool = False):
    return (256, 512) if small else (4096, 2048)


def c1_x(rows=4096, cols=2048, seed=0, r0=0, r1=None) -> np.ndarray:
    """Trained activation: bf16(N(0,1) with Bernoulli(1e-3) outliers x50)."""
    return f32_to_bf16_rne(normal_outliers_f32(rows, cols, seed, 0, 1e-3, 50.0, r0, r1))


def c1_rollout(rows=4096, cols=2048, seed=0, r0=0, r1=None) -> np.ndarray:
    """Rollout copy: bf16(fp32(x) + N(0, 1e-3^2)), noise from a second stream."""
    x = bf16_to_f32(c1_x(rows, cols, seed, r0, r1))
    e = noise_f32(rows, cols, seed, 1, 1e-3, r0, r1)
    return f32_to_bf16_rne(x + e)


# C2: MXFP4 MoE expert activations, Student-t(4)
def c2_shape(small: bool = False):
    return (512, 1024) if small else (16384, 4096)


def c2_pair(rows=16384, cols=4096, seed=1, r0=0, r1=None):
    """(trained, rollout): RNE and truncating bf16 roundings of the same fp32 draw."""
    t = student_t_f32(rows, cols, seed, 0, 4.0, r0, r1)
    return f32_to_bf16_rne(t), f32_to_bf16_rtz(t)


# C3: KV cache with per-channel magnitudes
def c3_shape(small: bool = False):
    tokens = 512 if small else 131072
    return tokens * 8, 128


def c3_channel_mag(seed=3, heads=8, dim=128) -> np.ndarray:
    g = _rng(seed, 99, 0)
    return np.exp(g.uniform(np.log(0.1), np.log(10.0), size=(heads, dim))).astype(np.float32)


def c3_kv(which: int, tokens=131072, heads=8, dim=128, seed=3, r0=0, r1=None) -> np.ndarray:
    """K (which=0) or V (which=1) as a (tokens*heads) x dim bf16 matrix; row = token*heads + head."""
    rows = tokens * heads
    r1 = rows if r1 is None else r1
    mag = c3_channel_mag(seed, heads, dim)
    x = normal_outliers_f32(rows, dim, seed, which, 0.0, 1.0, r0, r1)
    head = (np.arange(r0, r1) % heads)
    x *= mag[head]
    return f32_to_bf16_rne(x)


# C4: one deep layer of the guidance cache
C4_EXPERTS = 8
C4_W_SHAPE = (4096, 1536)
C4_A_SHAPE = (8192, 4096)
C4_LAYERS, C4_DEEP = 40, 20


def c4_tensors(layer: int, small: bool = False):
    """Yields (name, rows, cols, sigma, seed, stream) for the layer's tensors."""
    ws = (128, 96) if small else C4_W_SHAPE
    as_ = (256, 256) if small else C4_A_SHAPE
    seed = 1000 + layer
    for e in range(C4_EXPERTS):
        yield f"w{e}", ws[0], ws[1], 0.02, seed, 2 * e
    yield "act", as_[0], as_[1], 1.0, seed, 2 * C4_EXPERTS


def c4_pair(rows, cols, sigma, seed, stream, r0=0, r1=None):
    """(trained, rollout): bf16(N(0, sigma^2)) and bf16(x + N(0, (1e-3 sigma)^2))."""
    x = f32_to_bf16_rne(normal_outliers_f32(rows, cols, seed, stream, 0.0, 1.0, r0, r1, sigma=sigma))
    e = noise_f32(rows, cols, seed, stream + 1, 1e-3 * sigma, r0, r1)
    return x, f32_to_bf16_rne(bf16_to_f32(x) + e)


# C5: GEMM operand for the uniform grid + RHT16 + SR
def c5_shape(small: bool = False):
    return (256, 1024) if small else (65536, 8192)


def c5_x(rows=65536, cols=8192, seed=7, r0=0, r1=None) -> np.ndarray:
    return f32_to_bf16_rne(normal_outliers_f32(rows, cols, seed, 0, 5e-3, 30.0, r0, r1))


# Raw MXFP4 operand [rows, K]: codes uint8[rows*K/2], scales uint8[rows*K/32]
def mx_operand(rows: int, K: int, seed: int, stream: int, scale_lo: int = 118, scale_hi: int = 133,
               r0: int = 0, r1=None):
    r1 = rows if r1 is None else r1

    def codes(c, n):
        return _rng(seed, stream, c).integers(0, 256, (n, K // 2), dtype=np.uint8)

    def scales(c, n):
        return _rng(seed, stream + 1, c).integers(scale_lo, scale_hi + 1, (n, K // 32), dtype=np.uint8)
    return _gen(rows, K // 2, r0, r1, codes), _gen(rows, K // 32, r0, r1, scales)


# Matrix product workload: activations [8192, 4096] times one expert weight [1536 out, 4096 in]
GEMM_SHAPE = (8192, 1536, 4096)


C5_RHT_SEED = 7
C5_SR_SEED = 7
C2_SR_SEED = 1
