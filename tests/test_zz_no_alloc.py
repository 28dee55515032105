"""fp4_tensor_scale_noalloc (the tensor scale with the library's static workspace,
for callers that cannot allocate) equals fp4_tensor_scale_ws with a workspace of
the caller's, bit for bit, on two calls in a row, the second on a smaller input,
each called through the C ABI."""
import ctypes as C

import numpy as np
import pytest
import torch

from precision_rl_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from precision_rl_amd import fp4q
    fp4q.lib()
    return fp4q


def dev(u16, pad=0):
    rows, cols = u16.shape
    t = torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)
    if pad:
        buf = torch.zeros((rows, cols + pad), dtype=torch.bfloat16)
        buf[:, :cols] = t
        return buf.cuda()[:, :cols]
    return t.cuda()


def noalloc(fq, x, cfg, out):
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    c = cfg.c()
    st = fq.lib().fp4_tensor_scale_noalloc(C.byref(c), C.c_void_p(x.data_ptr()), rows, cols, ld,
                                           C.c_void_p(out.data_ptr()),
                                           C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fq.lib().fp4_last_error().decode()
    return out


def with_workspace(fq, x, cfg, ws, out):
    rows, cols = x.shape
    ld = x.stride(0) if rows > 1 else cols
    c = cfg.c()
    st = fq.lib().fp4_tensor_scale_ws(C.byref(c), C.c_void_p(x.data_ptr()), rows, cols, ld,
                                      C.c_void_p(out.data_ptr()), C.c_void_p(ws.data_ptr()), ws.numel(),
                                      C.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fq.lib().fp4_last_error().decode()
    return out


def bits(t):
    torch.cuda.synchronize()
    return np.float32(t.cpu().numpy()[0]).view(np.uint32)


@pytest.mark.parametrize("rht", [False, True])
def test_noalloc_equals_workspace_entry_point_twice(fq, rht):
    cfg = fq.Fp4Config(rht16=rht, rht_seed=5)
    ws = torch.zeros(fq.lib().fp4_tensor_scale_workspace_bytes(), dtype=torch.uint8, device="cuda")
    big = dev(W.c5_x(4096, 8192, seed=11))                 # the grid-stride launch, 1024 workgroups
    small = dev(W.c1_x(129, 96, seed=12), pad=8)           # one workgroup, padded rows
    for x in (big, small):
        a = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        b = torch.full((1,), -2.0, dtype=torch.float32, device="cuda")
        noalloc(fq, x, cfg, a)
        with_workspace(fq, x, cfg, ws, b)
        assert bits(a) == bits(b)
        assert bits(a) == bits(fq.fp4_tensor_scale(x, cfg))
