"""fp64 CPU oracle -- test infrastructure only (tests, smoke check, CPU baseline)."""
from .attention import (bf16_to_f64, reshape_and_cache, varlen_attention, merge_states,
                        merge_attn_states, cascade_attention, gather_kv)

__all__ = ["bf16_to_f64", "reshape_and_cache", "varlen_attention", "merge_states",
           "merge_attn_states", "cascade_attention", "gather_kv"]
