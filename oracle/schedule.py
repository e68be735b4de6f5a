"""The prefill and decode work items of a batch and their cost, from the attention mask, in
Python.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
use this module.

Source: the FA3 section of the vLLM FlashAttention page ("[vLLM] FlashAttention: IO-aware
타일링으로 ...") computes the distribution of the attention work before the kernel runs. The
pages do not define the items or their order; the readings here (also in the design notes):
  * a work item is one 256-row query tile of one prefill request (requests from num_decodes
    on), tile t holding query rows [256 t, min(256 (t + 1), query_len));
  * its cost is the number of 64-key tiles between the first and the last key any of its
    rows can see (the visible-key mask of the attention definition, see visible_keys);
  * the schedule lists every item once, costs non-increasing (longest first); items of equal
    cost may come in any order.
The decode items follow the split-KV reading of the RBLN "Attention 모드" page (overview: the
cache is processed partition by partition): the keys a decode row sees are cut at multiples
of the partition length P; an item is one partition holding at least one visible key,
numbered from the first such partition; its cost is its number of visible keys in 16-key
units, rounded up.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

from .naive_attention import visible_keys


def prefill_items(query_lens, seq_lens, num_decodes: int, causal: bool, window: int,
                  tile_rows: int = 256, tile_keys: int = 64) -> List[Tuple[int, int, int]]:
    """(request, q tile, cost) of every prefill work item, cost from the visible-key mask."""
    items = []
    for r in range(num_decodes, len(seq_lens)):
        ql, sl = int(query_lens[r]), int(seq_lens[r])
        if ql == 0:
            continue
        vis = visible_keys(ql, sl, causal, window)           # [ql, sl]
        for t in range(-(-ql // tile_rows)):
            rows = vis[t * tile_rows:(t + 1) * tile_rows]
            cols = np.nonzero(rows.any(axis=0))[0]
            cost = 0 if cols.size == 0 else int(cols[-1] // tile_keys - cols[0] // tile_keys + 1)
            items.append((r, t, cost))
    return items


def decode_items(seq_lens, num_decodes: int, window: int, part_tokens: int,
                 kv_skip: int = 0) -> List[Tuple[int, int, int]]:
    """(request, partition, cost) of every decode work item: request r < num_decodes sees, in
    this pass, the keys visible to its one query row among keys [kv_skip, seq_len), counted
    from kv_skip; cost = ceil(visible keys in the partition / 16)."""
    items = []
    for r in range(num_decodes):
        sl = int(seq_lens[r]) - kv_skip
        if sl <= 0:
            continue
        vis = np.nonzero(visible_keys(1, sl, True, window)[0])[0]
        parts = vis // part_tokens
        first = int(parts.min())
        for p in np.unique(parts):
            items.append((r, int(p) - first, int(-(-np.count_nonzero(parts == p) // 16))))
    return items
