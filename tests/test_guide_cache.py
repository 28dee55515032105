"""Guidance-cache registry: deep-layer policy and byte accounting (CPU), and the
rollout -> trainer round trip through the library (GPU, against the oracle)."""
import numpy as np
import pytest
import torch

from precision_rl_amd import guide_cache as G
from precision_rl_amd import fp4q as fq
from precision_rl_amd import workloads as W


def test_default_policy_is_the_later_half():
    c = G.GuideCache(num_layers=40)
    assert c.deep_layers == tuple(range(20, 40))
    assert not c.is_deep(19) and c.is_deep(20) and c.is_deep(39)
    with pytest.raises(ValueError):
        G.GuideCache(num_layers=4, deep_layers=(5,))


def test_byte_accounting_is_one_sixth_for_nvfp4():
    # per-tensor sizes of the C4 layer: guide on 20 layers vs full record on 40
    shapes = [W.C4_W_SHAPE] * W.C4_EXPERTS + [W.C4_A_SHAPE]
    guide = 20 * sum(G.guide_bytes(fq.NVFP4, r, c) - 4 for r, c in shapes)
    full = 40 * sum(G.full_record_bytes(fq.NVFP4, r, c) - 4 for r, c in shapes)
    assert guide * 6 == full
    assert guide == 314_572_800
    # MXFP4: 1.25 / 4.25 bits per element on half the layers
    r, c = W.C4_A_SHAPE
    ratio = (20 * (G.guide_bytes(fq.MXFP4, r, c))) / (40 * G.full_record_bytes(fq.MXFP4, r, c))
    assert abs(ratio - 1.25 / 4.25 / 2) < 1e-9


@pytest.mark.gpu
def test_rollout_to_trainer_round_trip_matches_oracle():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import oracle as O
    rows, cols = 64, 512
    cache = G.GuideCache(num_layers=4, deep_layers=(2, 3))
    oc = O.Cfg()
    for layer in range(4):
        xr_h = W.c1_rollout(rows, cols, seed=layer)
        x_h = W.c1_x(rows, cols, seed=layer)
        dev = lambda h: torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).cuda()
        codes, scales, ts = cache.rollout_quantize(layer, "act", dev(xr_h))
        gc, gs, ts_used, guided = cache.trainer_quantize(layer, "act", dev(x_h))
        assert guided == (layer >= 2)
        o_ts = O.tensor_scale(oc, xr_h)
        o_rc, o_rs, o_gb = O.quantize(oc, O.RTN, xr_h, o_ts, emit=True)
        assert (codes.cpu().numpy() == o_rc).all()
        if guided:
            want, _ = O.quantize(oc, O.GUIDED, x_h, o_ts, guide_bits=o_gb, guide_scales=o_rs)
        else:
            want, _ = O.quantize(oc, O.RTN, x_h, O.tensor_scale(oc, x_h))
        assert (gc.cpu().numpy() == want).all()
    assert len(cache) == 2
    assert cache.nbytes() == 2 * G.guide_bytes(fq.NVFP4, rows, cols)
