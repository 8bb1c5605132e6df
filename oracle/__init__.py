"""CPU fp64 attention oracle -- test infrastructure only (see oracle.c)."""
from .oracle import (attn_fwd, attn_rows, quantize_row, route_bit, words_per_row,  # noqa: F401
                     f16_to_f64, f64_to_f16_bits, round_f16, quantize_rows, attn_fwd_kv8,
                     attn_rows_kv8, e4m3_decode, e4m3_round, e4m3_encode, quantize_row_fp8)
