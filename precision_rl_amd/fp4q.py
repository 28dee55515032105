"""Thin ctypes binding of libfp4q (include/fp4q.h) over torch device tensors.

Argument marshalling only: shapes, strides, pointers and the current HIP
stream are passed to the C ABI, outputs are allocated with torch when the
caller does not provide them, and every computation runs in the library's
gfx950 kernels.  There is no fallback: if the library is missing or the
tensors are not on a GPU, the call raises.

Function names follow the C ABI (fp4_quantize, fp4_quantize_guided,
fp4_dequantize, guide_pack, guide_unpack, fp4_rht16, fp4_tensor_scale,
fp4_encode_values).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4q.so")

NVFP4, MXFP4 = 0, 1
E2M1, UNIFORM = 0, 1
RTN, SR = 0, 1
MODE_RTN, MODE_SR, MODE_GUIDED = 0, 1, 2
OUT_F32, OUT_BF16 = 0, 1


class Fp4Error(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        super().__init__(f"{where}: status {status}: {msg}")
        self.status = status


class _CCfg(C.Structure):
    _fields_ = [("format", C.c_int32), ("grid", C.c_int32), ("rounding", C.c_int32),
                ("rht16", C.c_int32), ("sr_seed", C.c_uint64), ("sr_offset", C.c_uint64),
                ("rht_seed", C.c_uint64), ("stream_out", C.c_int32)]


@dataclass
class Fp4Config:
    """Mirror of fp4_cfg."""
    format: int = NVFP4
    grid: int = E2M1
    rounding: int = RTN
    rht16: bool = False
    sr_seed: int = 0
    sr_offset: int = 0
    rht_seed: int = 0
    stream_out: bool = False    # outputs not read again soon: non-temporal stores

    @property
    def block(self) -> int:
        return 32 if self.format == MXFP4 else 16

    def c(self) -> _CCfg:
        """The C struct of these fields (shared by calls with equal fields; the library only reads it)."""
        key = (self.format, self.grid, self.rounding, int(bool(self.rht16)), self.sr_seed, self.sr_offset,
               self.rht_seed, int(bool(self.stream_out)))
        cc = _CFG_CACHE.get(key)
        if cc is None:
            if len(_CFG_CACHE) >= 4096:      # e.g. an SR offset that advances every step
                _CFG_CACHE.clear()
            cc = _CFG_CACHE[key] = _CCfg(*key)
        return cc


_CFG_CACHE: dict = {}


class _CTensor(C.Structure):
    _fields_ = [("x", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64), ("ld", C.c_int64),
                ("tensor_scale", C.c_void_p), ("codes", C.c_void_p), ("scales", C.c_void_p),
                ("guide_bits", C.c_void_p), ("guide_scales", C.c_void_p)]


MAX_GROUP = 16

_lib = None
EXPORTS = ("fp4_tensor_scale", "fp4_tensor_scale_ws", "fp4_tensor_scale_workspace_bytes",
           "fp4_quantize_with_tensor_scale",
           "fp4_tensor_scale_noalloc", "fp4_quantize", "fp4_quantize_guided", "fp4_quantize_grouped",
           "fp4_fake_quantize", "fp4_guide_mismatch", "fp4_dequantize", "guide_pack", "guide_pack_grouped",
           "guide_unpack",
           "fp4_gemm_mxfp4", "fp4_gemm_mxfp4_grouped", "fp4_gemm_mxfp4_quantize", "fp4_gemm_mxfp4_quantize_nvfp4",
           "fp4_rht16",
           "fp4_encode_values", "fp4_encode_scales", "fp4_stream_copy", "fp4_codes_bytes", "fp4_scales_bytes", "fp4_guide_bytes",
           "fp4_set_wait_limit", "fp4_status_str", "fp4_last_error")


class _CGuide(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64),
                ("guide_bits", C.c_void_p), ("guide_scales", C.c_void_p)]


class _CGemm(C.Structure):
    _fields_ = [("a_codes", C.c_void_p), ("a_scales", C.c_void_p), ("b_codes", C.c_void_p),
                ("b_scales", C.c_void_p), ("M", C.c_int64), ("N", C.c_int64), ("K", C.c_int64),
                ("c", C.c_void_p), ("ldc", C.c_int64)]


def lib():
    """Load libfp4q.so (built in-tree by ``precision_rl_amd/build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python precision_rl_amd/build.py` "
                          "(there is no CPU fallback)")
    L = C.CDLL(LIB_PATH)
    P, I64, I = C.c_void_p, C.c_int64, C.c_int
    CP = C.POINTER(_CCfg)
    sigs = {
        "fp4_tensor_scale": [CP, P, I64, I64, I64, P, P],
        "fp4_tensor_scale_ws": [CP, P, I64, I64, I64, P, P, C.c_size_t, P],
        "fp4_tensor_scale_noalloc": [CP, P, I64, I64, I64, P, P],
        "fp4_quantize": [CP, P, I64, I64, I64, P, P, P, P, P],
        "fp4_quantize_with_tensor_scale": [CP, P, I64, I64, I64, P, P, P, P, P, C.c_size_t, P, P],
        "fp4_quantize_guided": [CP, P, I64, I64, I64, P, P, P, P, P, P],
        "fp4_quantize_grouped": [CP, I, I, C.POINTER(_CTensor), P],
        "fp4_fake_quantize": [CP, I, P, I64, I64, I64, P, P, P, P, I64, P],
        "fp4_guide_mismatch": [CP, P, I64, I64, I64, P, P, P, P, P],
        "fp4_dequantize": [CP, P, P, P, I64, I64, P, I64, I, P],
        "guide_pack": [CP, P, P, I64, I64, P, P, P],
        "guide_pack_grouped": [CP, I, C.POINTER(_CGuide), P],
        "guide_unpack": [CP, P, P, I64, I64, P, P, P],
        "fp4_gemm_mxfp4": [P, P, P, P, I64, I64, I64, P, I64, I, P],
        "fp4_gemm_mxfp4_grouped": [I, C.POINTER(_CGemm), I, P],
        "fp4_gemm_mxfp4_quantize": [P, P, P, P, I64, I64, I64, P, P, P, P],
        "fp4_gemm_mxfp4_quantize_nvfp4": [P, P, P, P, I64, I64, I64, P, P, P, P, P],
        "fp4_rht16": [P, I64, I64, I64, C.c_uint64, I, P, I, P],
        "fp4_encode_values": [I, I, P, P, I64, P, P],
        "fp4_encode_scales": [P, I64, P, P],
        "fp4_stream_copy": [P, P, C.c_size_t, P],
    }
    for name, args in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = C.c_int
    L.fp4_set_wait_limit.argtypes = [C.c_uint32]
    L.fp4_set_wait_limit.restype = C.c_uint32
    L.fp4_tensor_scale_workspace_bytes.argtypes = []
    L.fp4_tensor_scale_workspace_bytes.restype = C.c_size_t
    for name in ("fp4_codes_bytes",):
        getattr(L, name).argtypes = [I64, I64]
        getattr(L, name).restype = C.c_size_t
    for name in ("fp4_scales_bytes", "fp4_guide_bytes"):
        getattr(L, name).argtypes = [I, I64, I64]
        getattr(L, name).restype = C.c_size_t
    L.fp4_status_str.argtypes = [I]
    L.fp4_status_str.restype = C.c_char_p
    L.fp4_last_error.argtypes = []
    L.fp4_last_error.restype = C.c_char_p
    _lib = L
    return L


def _check(status: int, where: str):
    if status != 0:
        raise Fp4Error(status, where, lib().fp4_last_error().decode())


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor) -> int:
    """The current HIP stream of t's device, as an address (ctypes passes ints as void*)."""
    if _raw_stream is not None:
        return _raw_stream(t.device.index)
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _on_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("fp4q tensors must be on a GPU device (no CPU path)")


def _matrix(x: torch.Tensor):
    """(rows, cols, ld) of a 2-D bf16 tensor with unit column stride."""
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("expected a 2-D bfloat16 tensor")
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        raise ValueError("the last dimension must be contiguous")
    ld = x.stride(0) if rows > 1 else cols
    return rows, cols, ld


def _alloc(shape, dtype, device) -> torch.Tensor:
    """Every output the binding allocates for a caller comes from here (uninitialised memory: the
    kernels write every element)."""
    return torch.empty(shape, dtype=dtype, device=device)


def _u8(n: int, like: torch.Tensor) -> torch.Tensor:
    return _alloc(n, torch.uint8, like.device)


# ---------------------------------------------------------------- entry points
def fp4_tensor_scale(x: torch.Tensor, cfg: Fp4Config, out: torch.Tensor | None = None) -> torch.Tensor:
    _on_gpu(x, out)
    rows, cols, ld = _matrix(x)
    out = _alloc(1, torch.float32, x.device) if out is None else out
    c = cfg.c()
    _check(lib().fp4_tensor_scale(C.byref(c), _ptr(x), rows, cols, ld, _ptr(out), _stream(x)),
           "fp4_tensor_scale")
    return out


def tensor_scale_workspace(device=None) -> torch.Tensor:
    """A zero-filled workspace for fp4_tensor_scale_ws (reusable by one stream of calls at a time)."""
    n = lib().fp4_tensor_scale_workspace_bytes()
    return torch.zeros(n, dtype=torch.uint8, device=device if device is not None else "cuda")


def fp4_tensor_scale_ws(x: torch.Tensor, cfg: Fp4Config, workspace: torch.Tensor,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """fp4_tensor_scale in one launch, with a workspace from tensor_scale_workspace()."""
    _on_gpu(x, workspace, out)
    rows, cols, ld = _matrix(x)
    out = _alloc(1, torch.float32, x.device) if out is None else out
    c = cfg.c()
    _check(lib().fp4_tensor_scale_ws(C.byref(c), _ptr(x), rows, cols, ld, _ptr(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), _stream(x)),
           "fp4_tensor_scale_ws")
    return out


def fp4_tensor_scale_noalloc(x: torch.Tensor, cfg: Fp4Config, out: torch.Tensor) -> torch.Tensor:
    """fp4_tensor_scale in one launch with the library's static workspace: nothing is allocated
    (out is required).  Calls that overlap on one GPU race."""
    _on_gpu(x, out)
    rows, cols, ld = _matrix(x)
    c = cfg.c()
    _check(lib().fp4_tensor_scale_noalloc(C.byref(c), _ptr(x), rows, cols, ld, _ptr(out), _stream(x)),
           "fp4_tensor_scale_noalloc")
    return out


def fp4_quantize(x: torch.Tensor, cfg: Fp4Config, tensor_scale: torch.Tensor | None = None,
                 emit: bool = False, codes=None, scales=None, bits=None):
    """Returns (codes, scales) or (codes, scales, guide_bits) when ``emit``."""
    _on_gpu(x, tensor_scale, codes, scales, bits)
    rows, cols, ld = _matrix(x)
    n = rows * cols
    codes = _u8(n // 2, x) if codes is None else codes
    scales = _u8(n // cfg.block, x) if scales is None else scales
    if emit and bits is None:
        bits = _u8(n // 8, x)
    c = cfg.c()
    _check(lib().fp4_quantize(C.byref(c), _ptr(x), rows, cols, ld, _ptr(tensor_scale), _ptr(codes),
                              _ptr(scales), _ptr(bits) if emit else None, _stream(x)), "fp4_quantize")
    return (codes, scales, bits) if emit else (codes, scales)


def fp4_quantize_with_tensor_scale(x: torch.Tensor, cfg: Fp4Config, workspace: torch.Tensor, emit: bool = False,
                                   ts=None, codes=None, scales=None, bits=None):
    """NVFP4 tensor scale and quantization together (one launch where the device holds the whole
    grid, else two), with a workspace from tensor_scale_workspace().  Returns (ts, codes, scales)
    or (ts, codes, scales, guide_bits) when ``emit``; the number of launches enqueued is kept in
    ``last_launches``."""
    global last_launches
    _on_gpu(x, workspace, ts, codes, scales, bits)
    rows, cols, ld = _matrix(x)
    n = rows * cols
    ts = _alloc(1, torch.float32, x.device) if ts is None else ts
    codes = _u8(n // 2, x) if codes is None else codes
    scales = _u8(n // cfg.block, x) if scales is None else scales
    if emit and bits is None:
        bits = _u8(n // 8, x)
    c = cfg.c()
    nl = C.c_int(0)
    _check(lib().fp4_quantize_with_tensor_scale(C.byref(c), _ptr(x), rows, cols, ld, _ptr(ts), _ptr(codes),
                                                _ptr(scales), _ptr(bits) if emit else None, _ptr(workspace),
                                                workspace.numel() * workspace.element_size(), C.byref(nl),
                                                _stream(x)), "fp4_quantize_with_tensor_scale")
    last_launches = nl.value
    return (ts, codes, scales, bits) if emit else (ts, codes, scales)


last_launches = 0


def fp4_quantize_guided(x: torch.Tensor, cfg: Fp4Config, guide_bits: torch.Tensor,
                        guide_scales: torch.Tensor, guide_tensor_scale: torch.Tensor | None = None,
                        codes=None, scales=None):
    _on_gpu(x, guide_bits, guide_scales, guide_tensor_scale, codes, scales)
    rows, cols, ld = _matrix(x)
    n = rows * cols
    codes = _u8(n // 2, x) if codes is None else codes
    scales = _u8(n // cfg.block, x) if scales is None else scales
    c = cfg.c()
    _check(lib().fp4_quantize_guided(C.byref(c), _ptr(x), rows, cols, ld, _ptr(guide_bits),
                                     _ptr(guide_scales), _ptr(guide_tensor_scale), _ptr(codes),
                                     _ptr(scales), _stream(x)), "fp4_quantize_guided")
    return codes, scales


def fp4_quantize_grouped(xs, cfg: Fp4Config, tensor_scales=None, emit: bool = False, guides=None,
                         outs=None):
    """Quantize up to MAX_GROUP tensors with one configuration in one launch.

    xs            list of 2-D bf16 device tensors
    tensor_scales list of f32[1] tensors (NVFP4; for guided, the guides' tensor scales)
    emit          RTN/SR: also return each tensor's guide bitplane
    guides        list of (guide_bits, guide_scales): guided quantization
    outs          optional list of (codes, scales[, bits]) output tensors
    Returns a list of (codes, scales) or (codes, scales, bits)."""
    n = len(xs)
    if not 1 <= n <= MAX_GROUP:
        raise ValueError(f"1..{MAX_GROUP} tensors per grouped call, got {n}")
    arr = (_CTensor * n)()
    results = []
    for t, x in enumerate(xs):
        _on_gpu(x)
        rows, cols, ld = _matrix(x)
        m = rows * cols
        if outs is not None:
            o = outs[t]
            codes, scales = o[0], o[1]
            bits = o[2] if len(o) > 2 else None
        else:
            codes, scales, bits = _u8(m // 2, x), _u8(m // cfg.block, x), None
        if emit and bits is None:
            bits = _u8(m // 8, x)
        ts = tensor_scales[t] if tensor_scales is not None else None
        gb = gs = None
        if guides is not None:
            gb, gs = guides[t]
        _on_gpu(codes, scales, bits, ts, gb, gs)
        arr[t] = _CTensor(x.data_ptr(), rows, cols, ld, ts.data_ptr() if ts is not None else None,
                          codes.data_ptr(), scales.data_ptr(),
                          (gb.data_ptr() if gb is not None else (bits.data_ptr() if emit else None)),
                          gs.data_ptr() if gs is not None else None)
        results.append((codes, scales, bits) if emit else (codes, scales))
    c = cfg.c()
    _check(lib().fp4_quantize_grouped(C.byref(c), int(guides is not None), n, arr, _stream(xs[0])),
           "fp4_quantize_grouped")
    return results


def fp4_fake_quantize(x: torch.Tensor, cfg: Fp4Config, tensor_scale: torch.Tensor | None = None,
                      guide_bits: torch.Tensor | None = None, guide_scales: torch.Tensor | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 dequantization of the quantized x in one pass (guided when a guide is given)."""
    _on_gpu(x, tensor_scale, guide_bits, guide_scales, out)
    rows, cols, ld = _matrix(x)
    if out is None:
        out = _alloc((rows, cols), torch.bfloat16, x.device)
    ld_out = out.stride(0) if rows > 1 else cols
    guided = guide_bits is not None
    c = cfg.c()
    _check(lib().fp4_fake_quantize(C.byref(c), int(guided), _ptr(x), rows, cols, ld, _ptr(tensor_scale),
                                   _ptr(guide_bits), _ptr(guide_scales), _ptr(out), ld_out, _stream(x)),
           "fp4_fake_quantize")
    return out


def fp4_guide_mismatch(x: torch.Tensor, cfg: Fp4Config, rollout_codes: torch.Tensor, rollout_scales: torch.Tensor,
                       tensor_scale: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Guided rounding of x with the rollout's full codes as the guide, compared with those codes.
    Returns a device int64[3]: elements counted, non-adjacent (|g| != |r|), mismatched (g != r)."""
    _on_gpu(x, rollout_codes, rollout_scales, tensor_scale, out)
    rows, cols, ld = _matrix(x)
    if out is None:
        out = _alloc(3, torch.int64, x.device)
    c = cfg.c()
    _check(lib().fp4_guide_mismatch(C.byref(c), _ptr(x), rows, cols, ld, _ptr(tensor_scale), _ptr(rollout_codes),
                                    _ptr(rollout_scales), _ptr(out), _stream(x)), "fp4_guide_mismatch")
    return out


def fp4_dequantize(codes: torch.Tensor, scales: torch.Tensor, cfg: Fp4Config, rows: int, cols: int,
                   tensor_scale: torch.Tensor | None = None, dtype=torch.bfloat16,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    _on_gpu(codes, scales, tensor_scale, out)
    if out is None:
        out = _alloc((rows, cols), dtype, codes.device)
    ld_out = out.stride(0) if rows > 1 else cols
    kind = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dequantize output must be bfloat16 or float32")
    c = cfg.c()
    _check(lib().fp4_dequantize(C.byref(c), _ptr(codes), _ptr(scales), _ptr(tensor_scale), rows, cols,
                                _ptr(out), ld_out, kind, _stream(codes)), "fp4_dequantize")
    return out


def fp4_gemm_mxfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
                   M: int, N: int, K: int, dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    """C[M, N] = A * B^T from the MXFP4 codes and scales of A [M, K] and B [N, K] (blocks along K)."""
    _on_gpu(a_codes, a_scales, b_codes, b_scales, out)
    if out is None:
        out = _alloc((M, N), dtype, a_codes.device)
    if out.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("gemm output must be bfloat16 or float32")
    ldc = out.stride(0) if M > 1 else N
    kind = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    _check(lib().fp4_gemm_mxfp4(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
                                _ptr(out), ldc, kind, _stream(a_codes)), "fp4_gemm_mxfp4")
    return out


def fp4_gemm_mxfp4_quantize(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
                            b_scales: torch.Tensor, M: int, N: int, K: int, emit: bool = True,
                            codes=None, scales=None, bits=None):
    """MXFP4 codes, scales (and guide bits) of the bf16-rounded C = A * B^T, quantized in the product's
    epilogue (C itself is not written).  Returns (codes, scales[, bits])."""
    _on_gpu(a_codes, a_scales, b_codes, b_scales, codes, scales, bits)
    n = M * N
    codes = _u8(n // 2, a_codes) if codes is None else codes
    scales = _u8(n // 32, a_codes) if scales is None else scales
    if emit and bits is None:
        bits = _u8(n // 8, a_codes)
    _check(lib().fp4_gemm_mxfp4_quantize(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
                                         _ptr(codes), _ptr(scales), _ptr(bits) if emit else None,
                                         _stream(a_codes)), "fp4_gemm_mxfp4_quantize")
    return (codes, scales, bits) if emit else (codes, scales)


def fp4_gemm_mxfp4_quantize_nvfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
                                  b_scales: torch.Tensor, M: int, N: int, K: int, tensor_scale: torch.Tensor,
                                  emit: bool = True, codes=None, scales=None, bits=None):
    """NVFP4 codes, E4M3 scales (and guide bits) of the bf16-rounded C = A * B^T under the tensor scale
    ``tensor_scale`` (f32[1] on the device), quantized in the product's epilogue.  Returns
    (codes, scales[, bits])."""
    _on_gpu(a_codes, a_scales, b_codes, b_scales, tensor_scale, codes, scales, bits)
    n = M * N
    codes = _u8(n // 2, a_codes) if codes is None else codes
    scales = _u8(n // 16, a_codes) if scales is None else scales
    if emit and bits is None:
        bits = _u8(n // 8, a_codes)
    _check(lib().fp4_gemm_mxfp4_quantize_nvfp4(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N,
                                               K, _ptr(tensor_scale), _ptr(codes), _ptr(scales),
                                               _ptr(bits) if emit else None, _stream(a_codes)),
           "fp4_gemm_mxfp4_quantize_nvfp4")
    return (codes, scales, bits) if emit else (codes, scales)


def fp4_gemm_mxfp4_grouped(products, dtype=torch.bfloat16, outs=None):
    """Several MXFP4 products in one call: products is a list of (a_codes, a_scales, b_codes, b_scales, M, N, K).
    Returns the list of C tensors (outs, or new [M, N] tensors of dtype)."""
    if not products:
        raise ValueError("no products")
    arr = (_CGemm * len(products))()
    res = []
    for i, (ac, asc, bc, bsc, M, N, K) in enumerate(products):
        _on_gpu(ac, asc, bc, bsc)
        out = outs[i] if outs is not None else _alloc((M, N), dtype, ac.device)
        _on_gpu(out)
        ldc = out.stride(0) if M > 1 else N
        arr[i] = _CGemm(_ptr(ac), _ptr(asc), _ptr(bc), _ptr(bsc), M, N, K, _ptr(out), ldc)
        res.append(out)
    if len({o.dtype for o in res}) != 1 or res[0].dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("grouped gemm outputs must all be bfloat16 or all float32")
    kind = OUT_BF16 if res[0].dtype == torch.bfloat16 else OUT_F32
    _check(lib().fp4_gemm_mxfp4_grouped(len(products), arr, kind, _stream(products[0][0])), "fp4_gemm_mxfp4_grouped")
    return res


def guide_pack(codes: torch.Tensor, scales: torch.Tensor, cfg: Fp4Config, rows: int, cols: int,
               bits=None, gscales=None):
    _on_gpu(codes, scales, bits, gscales)
    n = rows * cols
    bits = _u8(n // 8, codes) if bits is None else bits
    gscales = _u8(n // cfg.block, codes) if gscales is None else gscales
    c = cfg.c()
    _check(lib().guide_pack(C.byref(c), _ptr(codes), _ptr(scales), rows, cols, _ptr(bits), _ptr(gscales),
                            _stream(codes)), "guide_pack")
    return bits, gscales


def guide_pack_grouped(tensors, cfg: Fp4Config, outs=None):
    """guide_pack of several tensors in one launch: tensors is a list of (codes, scales, rows, cols).
    Returns the list of (guide_bits, guide_scales)."""
    if not tensors:
        raise ValueError("no tensors")
    arr = (_CGuide * len(tensors))()
    res = []
    for i, (codes, scales, rows, cols) in enumerate(tensors):
        _on_gpu(codes, scales)
        n = rows * cols
        if outs is not None:
            bits, gs = outs[i]
        else:
            bits, gs = _u8(n // 8, codes), _u8(n // cfg.block, codes)
        _on_gpu(bits, gs)
        arr[i] = _CGuide(_ptr(codes), _ptr(scales), rows, cols, _ptr(bits), _ptr(gs))
        res.append((bits, gs))
    c = cfg.c()
    _check(lib().guide_pack_grouped(C.byref(c), len(tensors), arr, _stream(tensors[0][0])), "guide_pack_grouped")
    return res


def guide_unpack(bits: torch.Tensor, gscales: torch.Tensor, cfg: Fp4Config, rows: int, cols: int,
                 mant=None, scales_out=None):
    _on_gpu(bits, gscales, mant, scales_out)
    n = rows * cols
    mant = _u8(n, bits) if mant is None else mant
    scales_out = _u8(n // cfg.block, bits) if scales_out is None else scales_out
    c = cfg.c()
    _check(lib().guide_unpack(C.byref(c), _ptr(bits), _ptr(gscales), rows, cols, _ptr(mant),
                              _ptr(scales_out), _stream(bits)), "guide_unpack")
    return mant, scales_out


def fp4_rht16(x: torch.Tensor, seed: int, inverse: bool = False, dtype=torch.float32,
              out: torch.Tensor | None = None) -> torch.Tensor:
    _on_gpu(x, out)
    rows, cols, ld = _matrix(x)
    out = _alloc((rows, cols), dtype, x.device) if out is None else out
    kind = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    _check(lib().fp4_rht16(_ptr(x), rows, cols, ld, seed, int(inverse), _ptr(out), kind, _stream(x)),
           "fp4_rht16")
    return out


def fp4_encode_values(v: torch.Tensor, grid: int, mode: int, aux: torch.Tensor | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    _on_gpu(v, aux, out)
    if v.dtype != torch.float32 or not v.is_contiguous():
        raise ValueError("v must be a contiguous float32 tensor")
    n = v.numel()
    out = _u8(n, v) if out is None else out
    _check(lib().fp4_encode_values(grid, mode, _ptr(v), _ptr(aux), n, _ptr(out), _stream(v)),
           "fp4_encode_values")
    return out


def fp4_encode_scales(t: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """E4M3 block-scale codes of the values t (>= 0, clamped to 448), round to nearest even."""
    _on_gpu(t, out)
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError("t must be a contiguous float32 tensor")
    n = t.numel()
    out = _u8(n, t) if out is None else out
    _check(lib().fp4_encode_scales(_ptr(t), n, _ptr(out), _stream(t)), "fp4_encode_scales")
    return out


def fp4_stream_copy(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Reference streaming copy of src's bytes into dst (same byte size, contiguous)."""
    _on_gpu(src, dst)
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("stream copy needs contiguous tensors of equal byte size")
    _check(lib().fp4_stream_copy(_ptr(src), _ptr(dst), nb, _stream(src)), "fp4_stream_copy")
    return dst


def codes_bytes(rows: int, cols: int) -> int:
    return lib().fp4_codes_bytes(rows, cols)


def scales_bytes(fmt: int, rows: int, cols: int) -> int:
    return lib().fp4_scales_bytes(fmt, rows, cols)


def guide_bytes(fmt: int, rows: int, cols: int) -> int:
    return lib().fp4_guide_bytes(fmt, rows, cols)
