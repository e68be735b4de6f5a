"""CPU oracle for exact softmax attention over a paged KV cache (test infrastructure).

This package is the ground truth that the HIP path is checked against. Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it; the library and its
Python binding never do. It shares no code with the HIP path.
"""
from .naive_attention import (attention, attend_rows, gather_kv, visible_keys,
                              softmax_weights, flops_visible_pairs)
from .cascade import cascade_attention, merge_partials
from .kv_write import kv_cache_write
from .fp8 import attention_fp8_kv, e4m3_quantize, e4m3_value
from .schedule import decode_items, prefill_items

__all__ = ["attention", "attend_rows", "gather_kv", "visible_keys", "softmax_weights",
           "flops_visible_pairs", "cascade_attention", "merge_partials", "kv_cache_write",
           "attention_fp8_kv", "e4m3_quantize", "e4m3_value", "prefill_items", "decode_items"]
