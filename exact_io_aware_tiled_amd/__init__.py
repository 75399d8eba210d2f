"""Exact IO-aware tiled softmax attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library built from ``csrc/`` (C ABI in
``include/eiat_attn.h``); ``attn`` is its Python binding.
"""
from .attn import (attn_bwd, attn_bwd_noalloc, attn_bwd_workspace_bytes, attn_decode,  # noqa: F401
                   attn_decode_workspace_bytes, attn_fwd, attn_fwd_fp8, attn_fwd_fp8_pv,
                   attn_quant_fp8, attn_quant_fp8_v, load_library)
