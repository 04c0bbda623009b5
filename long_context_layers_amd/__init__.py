"""Decayed causal linear attention (Lightning Attention) for AMD MI355X (gfx950).

The layer's kernels live in the HIP library ``lib/liblightning_attn.so``
(C ABI: ``include/lightning_attn.h``); this package is its thin binding.

    from long_context_layers_amd import prefill, decode_step
"""
from .binding import prefill, decode_step, load_library, status_string, LightningAttnError  # noqa: F401

__all__ = ["prefill", "decode_step", "load_library", "status_string", "LightningAttnError"]
