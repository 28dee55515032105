"""Reading the tensor-scale workspace after a call (test helper).

Layout, in 32-bit words: a 64-bit state word at word 0 (the epoch in word 0, in
word 1 the mark of the last launch whose wait gave up, 0 after a launch that did
not); sixteen copies of the one-launch fused form's published word (tag << 32 |
bits of s_t) from word 64, a 256-byte line apart; one 64-bit word per workgroup
from word 2048 (tag << 32 | bits of the workgroup's largest finite |y|).  Every
completed reduction advances the epoch by one and tags each of its workgroups'
words with the new epoch.
"""
import numpy as np
import torch

EPOCH, MARK, PUB, PUB_COPIES, LINE, GATHER = 0, 1, 64, 16, 64, 2048
TS_GROUPS_PER_WG, TS_MAX_WG = 1024, 1024      # one-launch tensor scale: groups per workgroup, grid cap
FUSED_GROUPS_PER_WG = 512                     # fused tensor scale + quantize


def words(ws):
    torch.cuda.synchronize()
    return ws.view(torch.int32).cpu().numpy().view(np.uint32).copy()


def epoch(ws):
    return int(words(ws)[EPOCH])


def mark(ws):
    return int(words(ws)[MARK])


def ts_grid(ngroups):
    return min(max(-(-ngroups // TS_GROUPS_PER_WG), 1), TS_MAX_WG)


def fused_grid(ngroups):
    return -(-ngroups // FUSED_GROUPS_PER_WG)


def check_after(ws, epoch_before, nwg, ts_bits=None, wg_max_bits=None, amax_bits=None):
    """The call advanced the epoch by one and tagged all nwg workgroup words with it;
    ts_bits: the published copies hold it under the same tag; wg_max_bits: each
    workgroup's own maximum; amax_bits: the largest of them."""
    w = words(ws)
    e = (epoch_before + 1) & 0xFFFFFFFF
    assert int(w[EPOCH]) == e, (int(w[EPOCH]), e)
    assert int(w[MARK]) == 0, "a completed call leaves no give-up mark"
    g = w[GATHER:GATHER + 2 * nwg].reshape(nwg, 2)        # little endian: (low, high)
    assert (g[:, 1] == e).all(), "a workgroup word without this call's tag"
    if ts_bits is not None:
        for c in range(PUB_COPIES):
            assert int(w[PUB + LINE * c + 1]) == e and int(w[PUB + LINE * c]) == int(ts_bits), c
    if wg_max_bits is not None:
        assert (g[:, 0] == np.asarray(wg_max_bits, dtype=np.uint32)).all(), "per-workgroup maxima"
    if amax_bits is not None:
        assert int(g[:, 0].max()) == int(amax_bits)


def chunk_max_bits(u16, elems_per_wg):
    """Largest finite |x| of each run of elems_per_wg elements of a bf16 tensor in
    row-major order, as the fp32 bits of that bf16 value."""
    flat = np.ascontiguousarray(u16).reshape(-1).astype(np.uint32) & 0x7FFF
    flat = np.where(flat < 0x7F80, flat, 0)
    n = -(-flat.size // elems_per_wg)
    pad = np.zeros(n * elems_per_wg, dtype=np.uint32)
    pad[:flat.size] = flat
    return pad.reshape(n, elems_per_wg).max(axis=1) << 16
