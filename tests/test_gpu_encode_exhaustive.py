"""Exhaustive check of the GPU element encode over every fp32 bit pattern.

The element encode is a step function of the scaled value v.  For each mode
the GPU encodes every non-NaN fp32 pattern of each sign (2^31 - 2^23 values,
in chunks generated on the device), and the positions where the code changes
are extracted on the GPU.  They must equal, exactly, the breakpoints the
definitions give in closed form:
  RTN     at each midpoint of adjacent codewords (the tie goes to the even code),
  guided  at the codewords themselves (a value on a codeword keeps it; between
          two codewords the one whose LSB is the guide bit),
  SR      at lo + (2u+1)/512 * gap in every bracket, for fixed random bytes u,
and the codes between breakpoints must be the expected ones.  The oracle is
evaluated at every breakpoint and its predecessor and must agree, so the GPU
function equals the oracle's on all 2^32 inputs except NaN patterns.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

CHUNK = 1 << 28
POS_END = 0x7F800000  # +inf (inclusive); NaN patterns above are not scanned


@pytest.fixture(scope="module")
def fq():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from precision_rl_amd import fp4q
    fp4q.lib()
    return fp4q


def bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def grid(g):
    return [Fraction(v) for v in ([0, 0.5, 1, 1.5, 2, 3, 4, 6] if g == 0 else range(8))]


def expected(g, mode, aux):
    """Closed-form (breakpoint pattern, code from that pattern on) for v >= 0, plus the code at 0."""
    G = grid(g)
    bp = []
    if mode == 0:  # RTN, ties to the even code
        for k in range(7):
            m = (G[k] + G[k + 1]) / 2
            p = bits(float(m))
            bp.append((p if (k + 1) % 2 == 0 else p + 1, k + 1))
        return 0, bp
    if mode == 2:  # guided with constant bit b
        b = aux & 1
        code = 0
        for k in range(1, 8):
            p = bits(float(G[k]))
            if (k & 1) == b:        # off-grid values just below G[k] already round up to k
                bp.append((bits(float(G[k - 1])) + 1, k))
            else:                   # G[k] itself is on the grid with LSB != b
                bp.append((p, k))
        bp.sort()
        return code, bp
    # SR with constant random byte u: up iff v > lo + (2u+1)/512 * gap
    u = aux & 0xFF
    for k in range(7):
        t = G[k] + Fraction(2 * u + 1, 512) * (G[k + 1] - G[k])
        bp.append((bits(float(t)) + 1, k + 1))
    return 0, bp


def gpu_breakpoints(fq, g, mode, aux, sign):
    """Code-change positions (bit patterns) over the scanned range of one sign, and codes there."""
    lo = 0x80000000 if sign else 0
    hi = lo + POS_END
    out_bp, out_code = [], []
    prev_last = None
    first_code = None
    for s in range(lo, hi + 1, CHUNK):
        e = min(s + CHUNK, hi + 1)
        m = e - s
        pad = (-m) % 8
        idx = torch.arange(s, e + pad, dtype=torch.int64, device="cuda")
        v = (idx & 0xFFFFFFFF).to(torch.int32).view(torch.float32)
        a = None
        if mode != 0:
            a = torch.full((m + pad,), aux, dtype=torch.uint8, device="cuda")
        c = fq.fp4_encode_values(v, g, mode, a)[:m]
        if first_code is None:
            first_code = int(c[0])
        if prev_last is not None and int(c[0]) != prev_last:
            out_bp.append(s)
            out_code.append(int(c[0]))
        ch = torch.nonzero(c[1:] != c[:-1]).flatten()
        if ch.numel():
            pos = (ch + 1).cpu().numpy()
            out_bp += [s + int(p) for p in pos]
            out_code += [int(x) for x in c[ch + 1].cpu().numpy()]
        prev_last = int(c[-1])
        del idx, v, c, a
    return first_code, list(zip(out_bp, out_code))


CASES = [(0, 0, 0), (1, 0, 0), (0, 2, 0), (0, 2, 1), (1, 2, 0), (1, 2, 1),
         (0, 1, 0), (0, 1, 1), (0, 1, 2), (0, 1, 64), (0, 1, 127), (0, 1, 128), (0, 1, 191), (0, 1, 254),
         (0, 1, 255), (1, 1, 0), (1, 1, 1), (1, 1, 127), (1, 1, 200), (1, 1, 255)]


@pytest.mark.parametrize("g,mode,aux", CASES)
@pytest.mark.parametrize("sign", [0, 1])
def test_encode_breakpoints_over_all_fp32(fq, g, mode, aux, sign):
    code0, exp = expected(g, mode, aux)
    first, got = gpu_breakpoints(fq, g, mode, aux, sign)
    s8 = 8 if sign else 0
    exp = [((p | (0x80000000 if sign else 0)), k | s8) for p, k in exp]
    assert first == (code0 | s8)
    assert got == exp, (got[:10], exp[:10])
    # the oracle agrees at every breakpoint and just before it
    for p, k in exp:
        v = struct.unpack("<f", struct.pack("<I", p))[0]
        vb = struct.unpack("<f", struct.pack("<I", p - 1))[0]
        assert (O.encode(g, mode, abs(v), aux) | s8) == k, hex(p)
        assert (O.encode(g, mode, abs(vb), aux) | s8) != k, hex(p - 1)


def test_e4m3_scale_encode_over_all_fp32_up_to_448(fq):
    # The NVFP4 block-scale code: E4M3FN round to nearest even of t in [0, 448]
    # (the kernels clamp t to 448 first).  The GPU encodes every fp32 pattern from
    # +0 to 448 and the code changes exactly at the midpoints of consecutive E4M3
    # values (a midpoint itself goes to the even code), which the oracle's decode
    # table gives; the oracle's encode agrees at every change and just before it.
    # Values above 448, infinity and NaN give the code of 448.
    hi = bits(448.0)
    got_bp, first = [], None
    prev_last = None
    for s in range(0, hi + 1, CHUNK):
        e = min(s + CHUNK, hi + 1)
        m = e - s
        pad = (-m) % 4
        idx = torch.arange(s, e + pad, dtype=torch.int64, device="cuda")
        v = (idx & 0xFFFFFFFF).to(torch.int32).view(torch.float32)
        c = fq.fp4_encode_scales(v)[:m]
        if first is None:
            first = int(c[0])
        if prev_last is not None and int(c[0]) != prev_last:
            got_bp.append((s, int(c[0])))
        ch = torch.nonzero(c[1:] != c[:-1]).flatten()
        if ch.numel():
            got_bp += [(s + int(p) + 1, int(k)) for p, k in zip(ch.cpu().numpy(), c[ch + 1].cpu().numpy())]
        prev_last = int(c[-1])
        del idx, v, c
    exp = []
    for code in range(0x7E):
        mid = (Fraction(O.e4m3_decode(code)) + Fraction(O.e4m3_decode(code + 1))) / 2
        p = bits(float(mid))
        assert Fraction(struct.unpack("<f", struct.pack("<I", p))[0]) == mid   # midpoints are exact fp32 values
        exp.append((p if (code + 1) % 2 == 0 else p + 1, code + 1))
    assert first == 0
    assert got_bp == exp, (got_bp[:6], exp[:6])
    for p, k in exp:
        v = struct.unpack("<f", struct.pack("<I", p))[0]
        vb = struct.unpack("<f", struct.pack("<I", p - 1))[0]
        assert O.e4m3_encode(v) == k and O.e4m3_encode(vb) == k - 1, hex(p)
    big = torch.tensor([448.0, 449.0, 464.0, 1e30, float("inf"), float("nan"), 3.4e38, 500.0], device="cuda")
    assert (fq.fp4_encode_scales(big).cpu().numpy() == 0x7E).all()
