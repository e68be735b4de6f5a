"""Writing the new tokens' K and V into the paged cache through slot_mapping, in numpy.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
use this module.

Source: vLLM FlashAttention page ("[vLLM] FlashAttention: IO-aware 타일링으로 ..."):
  * "FlashAttentionMetadata" section: slot_mapping is part of the batch metadata, next to
    block_table;
  * "왜 이 설계인가", item 2: through block_table and slot_mapping the kernels reach a KV cache
    that is not contiguous (PagedAttention);
  * "FlashAttentionBackend" section: cache shape (2, num_blocks, block_size, num_kv_heads,
    head_size), index 0 of the first axis is K, index 1 is V;
  * the DiffKV backend paragraph names the cache-write kernel (reshape_and_cache) that this
    step corresponds to.

Readings where the pages are silent (also listed in the design notes):
  * slot_mapping[t] is the flat slot of new token t: block slot // block_size, offset
    slot % block_size (the same block/offset split the block table uses for reads);
  * a negative slot marks a padding token that is not written;
  * the slots of one call are distinct (two tokens never target the same slot).
"""
from __future__ import annotations

import numpy as np


def kv_cache_write(kv_cache: np.ndarray, key: np.ndarray, value: np.ndarray,
                   slot_mapping: np.ndarray) -> np.ndarray:
    """Return a copy of kv_cache [2, num_blocks, block_size, num_kv_heads, head_size] with
    key[t] and value[t] ([num_tokens, num_kv_heads, head_size]) stored at slot_mapping[t]."""
    out = np.array(kv_cache, copy=True)
    block_size = out.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), block_size)
        out[0, blk, off] = key[t]
        out[1, blk, off] = value[t]
    return out
