"""MI355X (gfx950) fused attention forward (prefill) with TileMix FP16/INT8 routing.

The computation lives in the HIP library libattn_mi355x.so (C ABI in
include/attn.h); this package only marshals torch tensors into it.
"""
from ._lib import (AttnError, attn_abi_version, attn_debug_plan, attn_debug_quantize_rows,  # noqa: F401
                   attn_debug_route_dump, attn_fwd, attn_fwd_kv8, attn_fwd_kv8_stream, attn_fwd_lowp_stream,
                   attn_fwd_stream, attn_fwd_unfused, attn_last_error, attn_quantize_rows, load)

__all__ = ["AttnError", "attn_abi_version", "attn_debug_plan", "attn_debug_quantize_rows", "attn_debug_route_dump",
           "attn_fwd", "attn_fwd_kv8", "attn_fwd_kv8_stream", "attn_fwd_lowp_stream", "attn_fwd_stream",
           "attn_fwd_unfused",
           "attn_last_error", "attn_quantize_rows", "load"]
