"""fp64 CPU oracle -- test infrastructure only (tests, smoke check, CPU baseline)."""
from .attention import (bf16_to_f64, reshape_and_cache, varlen_attention, merge_states,
                        merge_attn_states, cascade_attention, gather_kv)
from .fp8 import e4m3_to_f64, f32_to_e4m3, quantize, reshape_and_cache_fp8, dequantize

__all__ = ["bf16_to_f64", "reshape_and_cache", "varlen_attention", "merge_states",
           "merge_attn_states", "cascade_attention", "gather_kv", "e4m3_to_f64", "f32_to_e4m3",
           "quantize", "reshape_and_cache_fp8", "dequantize"]
