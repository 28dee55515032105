"""Per-layer guidance cache: the rollout's compact quantization record, kept for
deep layers only, consumed by the trainer's guided quantization.

[TRACE-JA "量子化情報キャッシュ"] The rollout keeps, per quantization point,
the mantissa bit of the chosen codeword and the block scale (not the full
code), and only for the later layers (20 of 40 loses little; 10 or 5 lose
more); [TRACE-KO "작동 원리의 공학적 이해"] the trainer then rounds its own
values following that record.  This module is the host-side registry around
the library's guide_pack / fused emission / fp4_quantize_guided calls: it
decides which layers are deep, holds each (layer, tensor) guide on the GPU
and accounts for its bytes.  All computation goes through precision_rl_amd.fp4q.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import fp4q as fq


@dataclass
class GuideEntry:
    bits: object            # u8 bitplane, rows*cols/8 (device tensor)
    scales: object          # u8 block scales, rows*cols/B (device tensor)
    tensor_scale: object    # f32[1] NVFP4 tensor scale (device tensor) or None for MXFP4
    rows: int
    cols: int

    def nbytes(self) -> int:
        return (self.bits.numel() + self.scales.numel() +
                (4 if self.tensor_scale is not None else 0))


def guide_bytes(fmt: int, rows: int, cols: int) -> int:
    """Bytes of one tensor's guide: bitplane + scales (+ 4 for the NVFP4 tensor scale)."""
    b = 32 if fmt == fq.MXFP4 else 16
    return rows * cols // 8 + rows * cols // b + (4 if fmt == fq.NVFP4 else 0)


def full_record_bytes(fmt: int, rows: int, cols: int) -> int:
    """Bytes of the full quantization record it replaces: 4-bit codes + scales (+ tensor scale)."""
    b = 32 if fmt == fq.MXFP4 else 16
    return rows * cols // 2 + rows * cols // b + (4 if fmt == fq.NVFP4 else 0)


@dataclass
class GuideCache:
    """Registry of guides for the deep layers of a model.

    num_layers   total layers of the model (40 in the pages' ablation)
    deep_layers  layers that keep a guide; default: the later half
    cfg          quantizer configuration shared by rollout and trainer
    """
    num_layers: int = 40
    deep_layers: tuple | None = None
    cfg: fq.Fp4Config = field(default_factory=fq.Fp4Config)
    _entries: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.deep_layers is None:
            self.deep_layers = tuple(range(self.num_layers // 2, self.num_layers))
        bad = [l for l in self.deep_layers if not 0 <= l < self.num_layers]
        if bad:
            raise ValueError(f"deep layers out of range: {bad}")
        self.deep_layers = tuple(sorted(set(self.deep_layers)))

    # ------------------------------------------------------------ policy
    def is_deep(self, layer: int) -> bool:
        return layer in self.deep_layers

    # ------------------------------------------------------------ rollout side
    def rollout_quantize(self, layer: int, name: str, x, tensor_scale=None):
        """RTN quantize of a rollout tensor; for deep layers the guide bits are emitted in the
        same pass and recorded.  Returns (codes, scales, tensor_scale)."""
        if self.cfg.format == fq.NVFP4 and tensor_scale is None:
            tensor_scale = fq.fp4_tensor_scale(x, self.cfg)
        if self.is_deep(layer):
            codes, scales, bits = fq.fp4_quantize(x, self.cfg, tensor_scale, emit=True)
            rows, cols = x.shape
            self._entries[(layer, name)] = GuideEntry(bits, scales, tensor_scale, rows, cols)
        else:
            codes, scales = fq.fp4_quantize(x, self.cfg, tensor_scale)
        return codes, scales, tensor_scale

    def record(self, layer: int, name: str, codes, scales, tensor_scale, rows: int, cols: int):
        """Record the guide of an already quantized tensor (guide_pack); ignored for shallow layers."""
        if not self.is_deep(layer):
            return None
        bits, gscales = fq.guide_pack(codes, scales, self.cfg, rows, cols)
        e = GuideEntry(bits, gscales, tensor_scale, rows, cols)
        self._entries[(layer, name)] = e
        return e

    # ------------------------------------------------------------ trainer side
    def get(self, layer: int, name: str):
        return self._entries.get((layer, name))

    def trainer_quantize(self, layer: int, name: str, x, tensor_scale=None):
        """Guided quantize when a guide is recorded for (layer, name), plain RTN otherwise.
        Returns (codes, scales, tensor_scale_used, guided: bool)."""
        e = self.get(layer, name)
        if e is not None:
            if tuple(x.shape) != (e.rows, e.cols):
                raise ValueError(f"guide for {(layer, name)} has shape {(e.rows, e.cols)}, got {tuple(x.shape)}")
            codes, scales = fq.fp4_quantize_guided(x, self.cfg, e.bits, e.scales, e.tensor_scale)
            return codes, scales, e.tensor_scale, True
        cfg = fq.Fp4Config(format=self.cfg.format, grid=self.cfg.grid, rht16=self.cfg.rht16,
                           rht_seed=self.cfg.rht_seed)
        if cfg.format == fq.NVFP4 and tensor_scale is None:
            tensor_scale = fq.fp4_tensor_scale(x, cfg)
        codes, scales = fq.fp4_quantize(x, cfg, tensor_scale)
        return codes, scales, tensor_scale, False

    # ------------------------------------------------------------ accounting
    def nbytes(self) -> int:
        return sum(e.nbytes() for e in self._entries.values())

    def full_record_nbytes(self, all_layers: bool = True) -> int:
        """Bytes of the full codes+scales record for the same tensors on every layer
        (the naive transfer the cache replaces), assuming each layer holds the same tensors."""
        per_layer = {}
        for (layer, name), e in self._entries.items():
            per_layer.setdefault(name, e)
        one = sum(full_record_bytes(self.cfg.format, e.rows, e.cols) for e in per_layer.values())
        return one * (self.num_layers if all_layers else len(self.deep_layers))

    def clear(self):
        self._entries.clear()

    def __len__(self):
        return len(self._entries)
