"""Signal Field Attention (SFA) for AMD Instinct MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (include/sfa.h, libsfa.so):
  prefill      windowed softmax attention (last W <= 16 tokens) + far-field EWMA
  decode_step  one token for all layers with the W-slot ring cache
  enhance      optional triple-channel enhancement of an attention output
PyTorch supplies device memory and streams only.
"""
from .sfa import (PreparedPool, decode_step, decode_step_enhance, enhance, enhance_pool_bytes,  # noqa: F401
                  enhance_prepare_pool, enhance_prepared, enhance_workspace_size, prefill,
                  prefill_noalloc, prefill_workspace_size)
from ._lib import SFAError  # noqa: F401

__all__ = ["prefill", "prefill_noalloc", "decode_step", "decode_step_enhance", "enhance", "enhance_prepare_pool",
           "enhance_prepared", "enhance_pool_bytes", "PreparedPool", "prefill_workspace_size",
           "enhance_workspace_size", "SFAError"]
