"""Decayed causal linear attention (Lightning Attention) for AMD MI355X (gfx950).

The layer's kernels live in the HIP library ``lib/liblightning_attn.so``
(C ABI: ``include/lightning_attn.h``); this package is its thin binding.

    from long_context_layers_amd import prefill, prefill_varlen, decode_step, decode_multi
"""
from .binding import (prefill, prefill_varlen, prefill_varlen_walks, decode_step, decode_multi,  # noqa: F401
                      qk_norm_rope, prefill_qk_norm_rope, group_norm_gate, cp_fold, cp_correct,
                      prefill_workspace_bytes, prefill_f32_workspace_bytes, load_library, status_string,
                      LightningAttnError)

__all__ = ["prefill", "prefill_varlen", "prefill_varlen_walks", "decode_step", "decode_multi", "qk_norm_rope",
           "prefill_qk_norm_rope", "group_norm_gate", "cp_fold", "cp_correct", "prefill_workspace_bytes", "prefill_f32_workspace_bytes",
           "load_library", "status_string", "LightningAttnError"]
