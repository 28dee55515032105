"""MI355X-native block-scaled FP4 quantization (NVFP4 / MXFP4, RTN / SR /
rollout-guided rounding, guidance cache, RHT16, uniform grid).

The compute path is the C-ABI library ``libfp4q.so`` (hand-written gfx950 HIP
kernels); :mod:`precision_rl_amd.fp4q` is its thin ctypes binding over torch
device tensors.  Importing this package does not load the library.
"""
__all__ = ["fp4q", "workloads", "guide_cache"]
