"""The C-ABI library loads and exports every entry point its header declares;
argument errors are reported on the host before any launch (CPU only: none of
these calls reaches the GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4q.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in {"if", "defined"}))


@pytest.fixture(scope="module")
def fq():
    from precision_rl_amd import fp4q, build
    if build.stale():
        build.build()
    fq_lib = fp4q.lib()
    return fp4q


def test_header_declares_the_expected_calls():
    names = _declared()
    for n in ["fp4_quantize", "fp4_quantize_guided", "fp4_dequantize", "guide_pack", "guide_unpack", "fp4_guide_mismatch",
              "fp4_gemm_mxfp4", "fp4_gemm_mxfp4_grouped", "guide_pack_grouped", "fp4_rht16", "fp4_tensor_scale", "fp4_encode_values", "fp4_codes_bytes",
              "fp4_quantize_with_tensor_scale", "fp4_gemm_mxfp4_quantize", "fp4_gemm_mxfp4_quantize_nvfp4",
              "fp4_scales_bytes", "fp4_guide_bytes", "fp4_status_str", "fp4_last_error"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(fq):
    L = fq.lib()
    for n in _declared():
        assert hasattr(L, n), f"libfp4q.so does not export {n}"
    assert set(fq.EXPORTS) <= set(_declared())


def test_size_helpers(fq):
    assert fq.codes_bytes(4096, 2048) == 4096 * 2048 // 2
    assert fq.scales_bytes(fq.NVFP4, 4096, 2048) == 4096 * 2048 // 16
    assert fq.scales_bytes(fq.MXFP4, 16384, 4096) == 16384 * 4096 // 32
    assert fq.guide_bytes(fq.NVFP4, 16, 32) == 16 * 32 // 8 + 16 * 32 // 16 + 4


def _call_quantize(fq, cfg, x, rows, cols, ld, ts=16, codes=16, scales=16):
    L = fq.lib()
    c = cfg.c() if cfg is not None else None
    return L.fp4_quantize(C.byref(c) if c is not None else None, C.c_void_p(x), rows, cols, ld,
                          C.c_void_p(ts), C.c_void_p(codes), C.c_void_p(scales), None, None)


def test_host_side_argument_errors(fq):
    L = fq.lib()
    cfg = fq.Fp4Config()
    A = 1 << 20  # a fake, 16-byte-aligned address: never dereferenced, validation fails first
    assert _call_quantize(fq, None, A, 4, 32, 32) == 1
    assert "cfg" in L.fp4_last_error().decode()
    assert _call_quantize(fq, cfg, A, 4, 24, 24) == 2            # cols % 16
    assert _call_quantize(fq, fq.Fp4Config(format=fq.MXFP4), A, 4, 48, 48) == 2  # cols % 32
    assert _call_quantize(fq, cfg, A, 4, 32, 16) == 2            # ld < cols
    assert _call_quantize(fq, cfg, A, 4, 32, 36) == 3            # ld % 8
    assert _call_quantize(fq, cfg, A + 8, 4, 32, 32) == 3        # misaligned x
    assert _call_quantize(fq, cfg, 0, 4, 32, 32) == 1            # null x
    assert _call_quantize(fq, cfg, A, 4, 32, 32, ts=0) == 1      # NVFP4 needs a tensor scale
    assert _call_quantize(fq, cfg, A, -1, 32, 32) == 1
    assert _call_quantize(fq, fq.Fp4Config(format=7), A, 4, 32, 32) == 1
    assert _call_quantize(fq, fq.Fp4Config(rounding=3), A, 4, 32, 32) == 1
    assert _call_quantize(fq, cfg, A, 1 << 20, 1 << 16, 1 << 16) == 2   # too many elements
    # empty input is a no-op that succeeds without touching the device
    assert _call_quantize(fq, cfg, 0, 0, 32, 32) == 0
    assert _call_quantize(fq, cfg, 0, 5, 0, 0) == 0
    assert L.fp4_status_str(3).decode().startswith("misaligned")
    # encode_values: n % 8
    assert L.fp4_encode_values(0, 0, C.c_void_p(A), None, 12, C.c_void_p(A), None) == 2
    assert L.fp4_encode_values(0, 5, C.c_void_p(A), None, 16, C.c_void_p(A), None) == 1
    # dequantize: bad dtype and ld_out
    c = cfg.c()
    assert L.fp4_dequantize(C.byref(c), C.c_void_p(A), C.c_void_p(A), C.c_void_p(A), 4, 32,
                            C.c_void_p(A), 32, 9, None) == 1
    assert L.fp4_dequantize(C.byref(c), C.c_void_p(A), C.c_void_p(A), C.c_void_p(A), 4, 32,
                            C.c_void_p(A), 16, 0, None) == 2
    assert L.fp4_rht16(C.c_void_p(A), 4, 40, 40, 7, 0, C.c_void_p(A), 0, None) == 2
    # guide mismatch: counts pointer required and 8-byte aligned; shapes as for quantize
    gm = L.fp4_guide_mismatch
    assert gm(C.byref(c), C.c_void_p(A), 4, 32, 32, C.c_void_p(A), C.c_void_p(A), C.c_void_p(A), None, None) == 1
    assert gm(C.byref(c), C.c_void_p(A), 4, 32, 32, C.c_void_p(A), C.c_void_p(A), C.c_void_p(A),
              C.c_void_p(A + 4), None) == 3
    assert gm(C.byref(c), C.c_void_p(A), 4, 24, 24, C.c_void_p(A), C.c_void_p(A), C.c_void_p(A),
              C.c_void_p(A), None) == 2
    assert gm(C.byref(c), C.c_void_p(A), 4, 32, 32, None, C.c_void_p(A), C.c_void_p(A),
              C.c_void_p(A), None) == 1                   # NVFP4 needs the tensor scale


def test_gemm_host_side_errors(fq):
    g = fq.lib().fp4_gemm_mxfp4
    A = 1 << 20
    p = C.c_void_p(A)
    assert g(p, p, p, p, -1, 4, 64, p, 4, 0, None) == 1          # negative shape
    assert g(p, p, p, p, 4, 4, 48, p, 4, 0, None) == 2           # K % 32
    assert g(p, p, p, p, 4, 8, 64, p, 4, 0, None) == 2           # ldc < N
    assert g(p, p, p, p, 4, 4, 64, p, 4, 9, None) == 1           # unknown dtype
    assert g(None, p, p, p, 4, 4, 64, p, 4, 0, None) == 1        # null A codes
    assert g(p, p, p, None, 4, 4, 64, p, 4, 0, None) == 1        # null B scales
    assert g(C.c_void_p(A + 8), p, p, p, 4, 4, 64, p, 4, 0, None) == 3   # codes not 16-byte aligned
    assert g(p, p, p, p, 4, 4, 64, C.c_void_p(A + 2), 4, 0, None) == 3   # fp32 output not 4-byte aligned
    assert g(p, p, p, p, 1 << 31, 4, 64, p, 4, 0, None) == 2     # M too large
    # M == 0 or N == 0 is a no-op that touches nothing
    assert g(None, None, None, None, 0, 4, 64, None, 4, 0, None) == 0
    assert g(None, None, None, None, 4, 0, 64, None, 0, 1, None) == 0


def test_grouped_gemm_host_side_errors(fq):
    L = fq.lib()
    A = 1 << 20
    arr = (fq._CGemm * 17)()
    for i in range(17):
        arr[i] = fq._CGemm(A, A, A, A, 4, 4, 64, A, 4)
    g = L.fp4_gemm_mxfp4_grouped
    assert g(0, arr, 0, None) == 1
    assert g(17, arr, 0, None) == 1
    assert g(2, None, 0, None) == 1
    arr[1] = fq._CGemm(A, A, A, A, 4, 4, 48, A, 4)            # K % 32
    assert g(2, arr, 0, None) == 2
    assert "product 1" in L.fp4_last_error().decode()
    arr[1] = fq._CGemm(A, A, A, A, 4, 8, 64, A, 4)            # ldc < N
    assert g(2, arr, 0, None) == 2
    arr[0] = fq._CGemm(None, None, None, None, 0, 4, 64, None, 4)
    arr[1] = fq._CGemm(None, None, None, None, 4, 0, 64, None, 0)
    assert g(2, arr, 0, None) == 0                            # every product empty: nothing launched


def test_grouped_guide_pack_host_side_errors(fq):
    L = fq.lib()
    A = 1 << 20
    cfg = fq.Fp4Config().c()
    arr = (fq._CGuide * 17)()
    for i in range(17):
        arr[i] = fq._CGuide(A, A, 4, 32, A, A)
    g = L.guide_pack_grouped
    assert g(C.byref(cfg), 0, arr, None) == 1
    assert g(C.byref(cfg), 17, arr, None) == 1
    assert g(C.byref(cfg), 2, None, None) == 1
    arr[1] = fq._CGuide(A, A, 4, 24, A, A)               # cols % 16
    assert g(C.byref(cfg), 2, arr, None) == 2
    assert "tensor 1" in L.fp4_last_error().decode()
    arr[1] = fq._CGuide(A, None, 4, 32, A, A)            # null scales
    assert g(C.byref(cfg), 2, arr, None) == 1
    arr[0] = fq._CGuide(None, None, 0, 32, None, None)
    arr[1] = fq._CGuide(None, None, 4, 0, None, None)
    assert g(C.byref(cfg), 2, arr, None) == 0              # all empty: nothing launched


def test_binding_refuses_cpu_tensors(fq):
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fq.fp4_quantize(x, fq.Fp4Config(), torch.ones(1))


def test_grouped_host_side_errors(fq):
    L = fq.lib()
    A = 1 << 20
    cfg = fq.Fp4Config().c()
    arr = (fq._CTensor * 17)()
    for t in range(17):
        arr[t] = fq._CTensor(A, 4, 32, 32, A, A, A, None, None)
    assert L.fp4_quantize_grouped(C.byref(cfg), 0, 0, arr, None) == 1
    assert L.fp4_quantize_grouped(C.byref(cfg), 0, 17, arr, None) == 1
    assert L.fp4_quantize_grouped(C.byref(cfg), 0, 2, None, None) == 1
    arr[1] = fq._CTensor(A, 4, 24, 24, A, A, A, None, None)          # cols % 16
    assert L.fp4_quantize_grouped(C.byref(cfg), 0, 2, arr, None) == 2
    assert "tensor 1" in L.fp4_last_error().decode()
    arr[1] = fq._CTensor(A, 4, 32, 32, A, A, A, A, None)             # emission on one tensor only
    assert L.fp4_quantize_grouped(C.byref(cfg), 0, 2, arr, None) == 1
    arr[1] = fq._CTensor(A, 4, 32, 32, A, A, A, None, None)
    assert L.fp4_quantize_grouped(C.byref(cfg), 1, 2, arr, None) == 1  # guided needs guides


def test_tensor_scale_workspace_errors(fq):
    L = fq.lib()
    A = 1 << 20
    p = C.c_void_p(A)
    c = fq.Fp4Config().c()
    n = L.fp4_tensor_scale_workspace_bytes()
    assert n == 24576
    f = L.fp4_tensor_scale_ws
    assert f(C.byref(c), p, 4, 32, 32, p, None, n, None) == 1              # no workspace
    assert f(C.byref(c), p, 4, 32, 32, p, C.c_void_p(A + 16), n, None) == 3  # not 256-byte aligned
    assert f(C.byref(c), p, 4, 32, 32, p, p, n - 1, None) == 1              # too small
    assert "workspace" in L.fp4_last_error().decode()
    assert f(C.byref(c), p, 4, 24, 24, p, p, n, None) == 2                  # cols % 16
    assert f(C.byref(c), p, 4, 32, 32, None, p, n, None) == 1               # no output


def test_quantize_with_tensor_scale_host_side_errors(fq):
    L = fq.lib()
    A = 1 << 20
    p = C.c_void_p(A)
    n = L.fp4_tensor_scale_workspace_bytes()
    f = L.fp4_quantize_with_tensor_scale
    nl = C.c_int(-1)

    def call(cfg, cols=32, ts=p, ws=p, wsb=n, codes=p, scales=p):
        c = cfg.c()
        return f(C.byref(c), p, 4, cols, cols, ts, codes, scales, None, ws, wsb, C.byref(nl), None)

    ERR_ARG, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED = 1, 2, 3, 4
    assert call(fq.Fp4Config(format=fq.MXFP4)) == ERR_UNSUPPORTED      # MXFP4 has no tensor scale
    assert "NVFP4" in L.fp4_last_error().decode()
    assert call(fq.Fp4Config(), ws=None) == ERR_ARG
    assert call(fq.Fp4Config(), ws=C.c_void_p(A + 64)) == ERR_ALIGN
    assert call(fq.Fp4Config(), wsb=n - 1) == ERR_ARG
    assert call(fq.Fp4Config(), cols=24) == ERR_SHAPE
    assert call(fq.Fp4Config(), ts=None) == ERR_ARG
    assert call(fq.Fp4Config(), codes=None) == ERR_ARG
    assert call(fq.Fp4Config(), codes=C.c_void_p(A + 8)) == ERR_ALIGN
    assert nl.value == -1                                                 # nothing was launched


def test_gemm_quantize_host_side_errors(fq):
    g = fq.lib().fp4_gemm_mxfp4_quantize
    A = 1 << 20
    p = C.c_void_p(A)
    assert g(p, p, p, p, 64, 48, 512, p, p, p, None) == 2            # N % 32
    assert g(p, p, p, p, 64, 64, 544, p, p, p, None) == 4            # K not a multiple of 512
    assert g(p, p, p, p, 64, 64, 0, p, p, p, None) == 4              # K == 0
    assert g(p, p, p, p, 64, 64, 512, None, p, p, None) == 1         # no codes
    assert g(p, p, p, p, 64, 64, 512, C.c_void_p(A + 8), p, p, None) == 3   # misaligned codes
    assert g(p, p, p, p, 64, 64, 512, p, p, C.c_void_p(A + 4), None) == 3   # misaligned bits
    assert g(p, p, p, p, 0, 64, 512, None, None, None, None) == 0    # empty: no-op
    assert g(p, p, C.c_void_p(A + 1), p, 64, 64, 512, p, p, p, None) == 3   # misaligned B codes


def test_gemm_quantize_nvfp4_host_side_errors(fq):
    g = fq.lib().fp4_gemm_mxfp4_quantize_nvfp4
    A = 1 << 20
    p = C.c_void_p(A)
    assert g(p, p, p, p, 64, 64, 512, None, p, p, p, None) == 1               # no tensor scale
    assert g(p, p, p, p, 64, 64, 512, C.c_void_p(A + 2), p, p, p, None) == 3  # misaligned tensor scale
    assert g(p, p, p, p, 64, 48, 512, p, p, p, p, None) == 2                  # N % 32
    assert g(p, p, p, p, 64, 64, 544, p, p, p, p, None) == 4                  # K not a multiple of 512
    assert g(p, p, p, p, 64, 64, 512, p, p, C.c_void_p(A + 1), p, None) == 3  # scales: two bytes per store
    assert g(p, p, p, p, 64, 64, 512, p, None, p, p, None) == 1               # no codes
    assert g(p, p, p, p, 0, 64, 512, p, None, None, None, None) == 0          # empty: no-op


def test_cfg_layout_and_stream_out_values(fq):
    # the binding's struct matches the header's 48-byte fp4_cfg, and stream_out takes 0 or 1 only
    assert C.sizeof(fq._CCfg) == 48
    assert fq._CCfg.stream_out.offset == 40
    L = fq.lib()
    A = 1 << 20
    p = C.c_void_p(A)
    for v, want in ((0, 0), (1, 0), (2, 1), (-1, 1)):
        c = fq.Fp4Config(format=fq.MXFP4).c()
        c2 = fq._CCfg(c.format, c.grid, c.rounding, c.rht16, c.sr_seed, c.sr_offset, c.rht_seed, v)
        st = L.fp4_quantize(C.byref(c2), p, 0, 32, 32, None, p, p, None, None)   # empty: checks only
        assert st == want, (v, st)


def test_wait_limit_setter(fq):
    L = fq.lib()
    prev = L.fp4_set_wait_limit(7)
    try:
        assert prev == 1 << 20
        assert L.fp4_set_wait_limit(0) == 7
    finally:
        assert L.fp4_set_wait_limit(prev) == 0
