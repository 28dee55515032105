"""Straight-through fake quantization for QAT (torch.autograd wrappers).

[TRACE-JA "TRACEの仕組み"] The trainer's forward pass uses the quantized value
chosen (guided by the rollout for deep layers) and the backward pass uses the
straight-through estimator: the gradient flows through the quantized value as
if quantization were the identity.  Forward runs fp4_fake_quantize in the
library; backward returns the incoming gradient unchanged.
"""
from __future__ import annotations

import torch

from . import fp4q as fq


class _FakeQuantSTE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, cfg, tensor_scale, guide_bits, guide_scales):
        return fq.fp4_fake_quantize(x, cfg, tensor_scale, guide_bits, guide_scales)

    @staticmethod
    def backward(ctx, grad_out):
        return grad_out, None, None, None, None


def fake_quantize_ste(x: torch.Tensor, cfg: fq.Fp4Config, tensor_scale: torch.Tensor | None = None,
                      guide_bits: torch.Tensor | None = None,
                      guide_scales: torch.Tensor | None = None) -> torch.Tensor:
    """Quantize-dequantize x (bf16, 2-D) in the forward pass, identity gradient backward.
    Without a guide it rounds per cfg.rounding; with (guide_bits, guide_scales[, tensor_scale
    of the guide]) it reproduces the rollout's rounding choices."""
    if cfg.format == fq.NVFP4 and tensor_scale is None:
        if guide_bits is not None:
            raise ValueError("guided NVFP4 fake quantization needs the guide's tensor scale")
        tensor_scale = fq.fp4_tensor_scale(x.detach(), cfg)
    return _FakeQuantSTE.apply(x, cfg, tensor_scale, guide_bits, guide_scales)
