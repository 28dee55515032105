"""CPU oracle for block-scaled FP4 quantization (ctypes over libfp4_oracle.so).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``precision_rl_amd``) never imports it.

Every function takes and returns numpy arrays in the same layouts as the
product library: bf16 tensors as ``uint16`` bit patterns (row-major, row
stride ``ld`` elements), packed codes ``uint8[rows*cols/2]`` (element i in
nibble i%2 of byte i/2), scales ``uint8[rows*cols/B]``, guide bitplanes
``uint8[rows*cols/8]`` (bit i%8 of byte i/8).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

NVFP4, MXFP4 = 0, 1
E2M1, UNIFORM = 0, 1
RTN, SR, GUIDED = 0, 1, 2


class OrcCfg(C.Structure):
    _fields_ = [("format", C.c_int32), ("grid", C.c_int32), ("rht16", C.c_int32),
                ("reserved", C.c_int32), ("rht_seed", C.c_uint64), ("sr_seed", C.c_uint64),
                ("sr_offset", C.c_uint64)]


@dataclass
class Cfg:
    format: int = NVFP4
    grid: int = E2M1
    rht16: bool = False
    rht_seed: int = 0
    sr_seed: int = 0
    sr_offset: int = 0

    @property
    def block(self) -> int:
        return 32 if self.format == MXFP4 else 16

    def c(self) -> OrcCfg:
        return OrcCfg(self.format, self.grid, int(bool(self.rht16)), 0, self.rht_seed, self.sr_seed,
                      self.sr_offset)


_lib = None


def lib():
    global _lib
    if _lib is None:
        # FP4Q_ORACLE_LIB names another build of the same source; the mutation
        # tests point it at copies with a planted mistake to show the pins fail.
        path = os.environ.get("FP4Q_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = C.CDLL(path)
        P = C.c_void_p
        I64 = C.c_int64
        F = C.c_float
        L.orc_mul32.restype = F; L.orc_mul32.argtypes = [F, F]
        L.orc_div32.restype = F; L.orc_div32.argtypes = [F, F]
        L.orc_add32.restype = F; L.orc_add32.argtypes = [F, F]
        L.orc_sub32.restype = F; L.orc_sub32.argtypes = [F, F]
        L.orc_grid.restype = C.c_double; L.orc_grid.argtypes = [C.c_int, C.c_int]
        L.orc_e4m3_decode.restype = C.c_double; L.orc_e4m3_decode.argtypes = [C.c_uint]
        L.orc_e4m3_encode.restype = C.c_uint; L.orc_e4m3_encode.argtypes = [F]
        L.orc_e8m0_decode.restype = C.c_double; L.orc_e8m0_decode.argtypes = [C.c_uint]
        L.orc_philox4x32_10.restype = None; L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_rht_signs.restype = C.c_uint32; L.orc_rht_signs.argtypes = [C.c_uint64]
        L.orc_rht16_vec.restype = None; L.orc_rht16_vec.argtypes = [P, C.c_uint32, C.c_int, P]
        L.orc_rht16.restype = None
        L.orc_rht16.argtypes = [P, I64, I64, I64, C.c_uint64, C.c_int, C.c_int, P]
        L.orc_tensor_scale.restype = F
        L.orc_tensor_scale.argtypes = [C.POINTER(OrcCfg), P, I64, I64, I64]
        L.orc_block_params.restype = None
        L.orc_block_params.argtypes = [C.POINTER(OrcCfg), F, F, C.POINTER(C.c_uint), C.POINTER(F)]
        L.orc_encode.restype = C.c_uint; L.orc_encode.argtypes = [C.c_int, C.c_int, F, C.c_uint]
        L.orc_quantize.restype = C.c_int
        L.orc_quantize.argtypes = [C.POINTER(OrcCfg), C.c_int, P, I64, I64, I64, I64, F, P, P, P, P, P]
        L.orc_dequantize.restype = None
        L.orc_dequantize.argtypes = [C.POINTER(OrcCfg), P, P, F, I64, I64, C.c_int, P]
        L.orc_guide_pack.restype = None
        L.orc_guide_pack.argtypes = [C.POINTER(OrcCfg), P, P, I64, I64, P, P]
        L.orc_guide_unpack.restype = None
        L.orc_guide_unpack.argtypes = [C.POINTER(OrcCfg), P, P, I64, I64, P, P]
        L.orc_guide_mismatch.restype = C.c_int
        L.orc_guide_mismatch.argtypes = [C.POINTER(OrcCfg), P, I64, I64, I64, F, P, P, P]
        L.orc_gemm_mx.restype = C.c_int
        L.orc_gemm_mx.argtypes = [P, P, P, P, I64, I64, I64, P, P]
        L.orc_encode_many.restype = None
        L.orc_encode_many.argtypes = [C.c_int, C.c_int, P, P, P, I64]
        L.orc_encode_breakpoints.restype = I64
        L.orc_encode_breakpoints.argtypes = [C.c_int, C.c_int, C.c_uint, C.c_uint32, C.c_uint32, P, I64]
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 1
    return a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- scalars
def mul32(a, b): return lib().orc_mul32(a, b)
def div32(a, b): return lib().orc_div32(a, b)
def add32(a, b): return lib().orc_add32(a, b)
def sub32(a, b): return lib().orc_sub32(a, b)
def grid_value(grid: int, k: int) -> float: return lib().orc_grid(grid, k)
def e4m3_decode(code: int) -> float: return lib().orc_e4m3_decode(code)
def e4m3_encode(t: float) -> int: return lib().orc_e4m3_encode(t)
def e8m0_decode(code: int) -> float: return lib().orc_e8m0_decode(code)
def encode(grid: int, mode: int, v: float, aux: int = 0) -> int: return lib().orc_encode(grid, mode, v, aux)
def rht_signs(seed: int) -> int: return lib().orc_rht_signs(seed)


def philox4x32_10(ctr, key) -> tuple:
    c = (C.c_uint32 * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
    k = (C.c_uint32 * 2)(*[int(x) & 0xFFFFFFFF for x in key])
    o = (C.c_uint32 * 4)()
    lib().orc_philox4x32_10(C.cast(c, C.c_void_p), C.cast(k, C.c_void_p), C.cast(o, C.c_void_p))
    return tuple(o)


def block_params(cfg: Cfg, amax: float, ts: float = 1.0):
    code = C.c_uint()
    inv = C.c_float()
    cc = cfg.c()
    lib().orc_block_params(C.byref(cc), amax, ts, C.byref(code), C.byref(inv))
    return code.value, inv.value


def rht16_vec(x: np.ndarray, signs: int, inverse: bool = False) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(16, dtype=np.float32)
    lib().orc_rht16_vec(_p(x), signs, int(inverse), _p(y))
    return y


# ---------------------------------------------------------------- tensors
def _bf16_2d(x: np.ndarray, cols: int | None = None):
    x = np.asarray(x)
    assert x.dtype == np.uint16, "bf16 inputs are uint16 bit patterns"
    if x.ndim == 1:
        assert cols is not None
        x = x.reshape(-1, cols)
    rows, ld = x.shape
    return x, rows, ld


def tensor_scale(cfg: Cfg, x: np.ndarray, cols: int | None = None) -> float:
    x, rows, ld = _bf16_2d(x, cols)
    cols = ld if cols is None else cols
    xc = np.ascontiguousarray(x)
    cc = cfg.c()
    return lib().orc_tensor_scale(C.byref(cc), _p(xc), rows, cols, ld)


def quantize(cfg: Cfg, mode: int, x: np.ndarray, ts: float = 1.0, cols: int | None = None,
             row0: int = 0, guide_bits: np.ndarray | None = None,
             guide_scales: np.ndarray | None = None, emit: bool = False):
    """Quantize the rows of ``x`` (uint16[rows, ld], the first ``cols`` columns used),
    which are rows ``row0 ..`` of the whole tensor.  Returns (codes, scales[, bits])."""
    x, rows, ld = _bf16_2d(x, cols)
    cols = ld if cols is None else cols
    xc = np.ascontiguousarray(x)
    B = cfg.block
    n = rows * cols
    codes = np.zeros(n // 2, dtype=np.uint8)
    scales = np.zeros(n // B, dtype=np.uint8)
    bits = np.zeros(n // 8, dtype=np.uint8) if emit else None
    gb = np.ascontiguousarray(guide_bits, dtype=np.uint8) if guide_bits is not None else None
    gs = np.ascontiguousarray(guide_scales, dtype=np.uint8) if guide_scales is not None else None
    if mode == GUIDED:
        assert gb is not None and gs is not None
        assert gb.size >= n // 8 and gs.size >= n // B
    cc = cfg.c()
    rc = lib().orc_quantize(C.byref(cc), mode, _p(xc), row0, rows, cols, ld, ts, _p(gb), _p(gs),
                            _p(codes), _p(scales), _p(bits))
    if rc != 0:
        raise ValueError("oracle quantize: bad shape")
    return (codes, scales, bits) if emit else (codes, scales)


def dequantize(cfg: Cfg, codes: np.ndarray, scales: np.ndarray, ts: float, rows: int, cols: int,
               out_bf16: bool = False) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty(rows * cols, dtype=np.uint16 if out_bf16 else np.float32)
    cc = cfg.c()
    lib().orc_dequantize(C.byref(cc), _p(codes), _p(scales), ts, rows, cols, int(out_bf16), _p(out))
    return out


def guide_pack(cfg: Cfg, codes: np.ndarray, scales: np.ndarray, rows: int, cols: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    n = rows * cols
    bits = np.empty(n // 8, dtype=np.uint8)
    gs = np.empty(n // cfg.block, dtype=np.uint8)
    cc = cfg.c()
    lib().orc_guide_pack(C.byref(cc), _p(codes), _p(scales), rows, cols, _p(bits), _p(gs))
    return bits, gs


def guide_unpack(cfg: Cfg, bits: np.ndarray, gscales: np.ndarray, rows: int, cols: int):
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    gscales = np.ascontiguousarray(gscales, dtype=np.uint8)
    n = rows * cols
    mant = np.empty(n, dtype=np.uint8)
    so = np.empty(n // cfg.block, dtype=np.uint8)
    cc = cfg.c()
    lib().orc_guide_unpack(C.byref(cc), _p(bits), _p(gscales), rows, cols, _p(mant), _p(so))
    return mant, so


def rht16(x: np.ndarray, seed: int, inverse: bool = False, out_bf16: bool = False,
          cols: int | None = None) -> np.ndarray:
    x, rows, ld = _bf16_2d(x, cols)
    cols = ld if cols is None else cols
    xc = np.ascontiguousarray(x)
    out = np.empty(rows * cols, dtype=np.uint16 if out_bf16 else np.float32)
    lib().orc_rht16(_p(xc), rows, cols, ld, seed, int(inverse), int(out_bf16), _p(out))
    return out


def encode_many(grid: int, mode: int, v: np.ndarray, aux: np.ndarray | None = None) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32).ravel()
    a = None if aux is None else np.ascontiguousarray(np.broadcast_to(aux, v.shape), dtype=np.uint32)
    out = np.empty(v.size, dtype=np.uint8)
    lib().orc_encode_many(grid, mode, _p(v), _p(a), _p(out), v.size)
    return out


def encode_breakpoints(grid: int, mode: int, aux: int, lo: int, hi: int, cap: int = 1 << 16):
    out = np.empty(cap, dtype=np.uint32)
    n = lib().orc_encode_breakpoints(grid, mode, aux, lo, hi, _p(out), cap)
    return out[:min(n, cap)].copy(), n


def guide_mismatch(cfg: Cfg, x: np.ndarray, ts: float, rollout_codes: np.ndarray, rollout_scales: np.ndarray,
                   cols: int | None = None) -> tuple:
    """(elements, non-adjacent, mismatched) of 1-bit guided rounding against the rollout's full codes."""
    x, rows, ld = _bf16_2d(x, cols)
    cols = ld if cols is None else cols
    xc = np.ascontiguousarray(x)
    out = np.zeros(3, dtype=np.uint64)
    cc = cfg.c()
    rc = lib().orc_guide_mismatch(C.byref(cc), _p(xc), rows, cols, ld, ts,
                                  _p(np.ascontiguousarray(rollout_codes, np.uint8)),
                                  _p(np.ascontiguousarray(rollout_scales, np.uint8)), _p(out))
    if rc:
        raise ValueError(f"orc_guide_mismatch failed ({rc})")
    return tuple(int(v) for v in out)


def gemm_mx(a_codes: np.ndarray, a_scales: np.ndarray, b_codes: np.ndarray, b_scales: np.ndarray,
            M: int, N: int, K: int) -> tuple:
    """MXFP4 product A * B^T in float64: returns (C[M, N], sum_k |a b| [M, N]).

    A is [M, K] and B is [N, K], each given as the codes and scales the MXFP4
    quantizer writes for a row-major tensor (blocks of 32 along K)."""
    ac = np.ascontiguousarray(a_codes, np.uint8).ravel()
    asc = np.ascontiguousarray(a_scales, np.uint8).ravel()
    bc = np.ascontiguousarray(b_codes, np.uint8).ravel()
    bsc = np.ascontiguousarray(b_scales, np.uint8).ravel()
    assert ac.size >= M * K // 2 and asc.size >= M * K // 32
    assert bc.size >= N * K // 2 and bsc.size >= N * K // 32
    c = np.empty((M, N), dtype=np.float64)
    mag = np.empty((M, N), dtype=np.float64)
    if lib().orc_gemm_mx(_p(ac), _p(asc), _p(bc), _p(bsc), M, N, K, _p(c), _p(mag)):
        raise ValueError("oracle gemm: K must be a multiple of 32 (or out of memory)")
    return c, mag
