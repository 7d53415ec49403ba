"""MI355X (gfx950) library for the frozen-NF4 linear layer with a LoRA adapter.

The computation lives in libqlora_nf4.so (HIP kernels behind a C ABI, see
include/qlora_nf4.h); this package is its thin Python binding.
"""
from .api import (NF4Weight, qlora_adamw_step, qlora_adamw_step16, qlora_dropout_mask,
                  qlora_dropout_mask_bytes, qlora_linear_bwd, qlora_linear_bwd_dropout,
                  qlora_linear_fwd, qlora_linear_fwd_dropout, qlora_linear_fwd_noalloc,
                  qlora_linear_workspace,
                  qlora_linear_workspace_dropout, qlora_nf4_dequantize, qlora_nf4_merge,
                  qlora_nf4_quantize, qlora_pre_dequant_min_tokens,
                  qlora_set_pre_dequant_min_tokens)
from ._lib import QloraError

__all__ = ["NF4Weight", "QloraError", "qlora_nf4_quantize", "qlora_nf4_dequantize",
           "qlora_nf4_merge", "qlora_linear_fwd", "qlora_linear_bwd", "qlora_linear_workspace",
           "qlora_adamw_step", "qlora_adamw_step16", "qlora_dropout_mask", "qlora_dropout_mask_bytes",
           "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout",
           "qlora_linear_workspace_dropout", "qlora_linear_fwd_noalloc",
           "qlora_set_pre_dequant_min_tokens", "qlora_pre_dequant_min_tokens"]
