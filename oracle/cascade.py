"""Cascade attention over a common prefix, in fp64, following the steps the pages give.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
use this module.

Source: vLLM FlashAttention page ("[vLLM] FlashAttention: IO-aware 타일링으로 ..."), section
"Cascade Attention: 공통 프리픽스 최적화", and the use_cascade / common_prefix_len fields of its
"FlashAttentionMetadata" section. When every request of a batch starts with the same prefix,
the prefix part of attention is computed once for the whole batch and each request's own
suffix separately:
  1. prefix pass: a batch of one sequence whose queries are all the batch's query tokens and
     whose keys are the common prefix (its seq len is common_prefix_len), not causal;
  2. suffix pass: every request over its keys after the prefix (seq len reduced by
     common_prefix_len), causal as the batch is;
  3. each query row's two partial results are combined through their log-sum-exps, the same
     combination of partial softmax results that the RBLN "Attention 모드" page (Overview)
     describes for KV partitions.
Because the method is exact, the result equals plain attention over all keys; the pins
check this decomposition against ``attention`` and check the merge on its own.

Readings where the page is silent (also listed in the design notes):
  * the prefix is a whole number of cache blocks (common_prefix_len % block_size == 0) and
    its blocks are the first common_prefix_len / block_size entries of every block-table row;
  * every query sits after the prefix (common_prefix_len <= context_len of every request),
    so each query sees every prefix key and the prefix pass needs no mask;
  * suffix positions keep the batch's bottom-right causal alignment (seq len and context
    length both shrink by common_prefix_len);
  * no sliding window (a window could cut into the prefix).
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .naive_attention import attention


def merge_partials(outs: Sequence[np.ndarray], lses: Sequence[np.ndarray]
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial attention results over disjoint key sets.

    outs[i] [..., d] is the softmax-weighted mean of V over key set i and lses[i] [...] the
    natural-log log-sum-exp of the scaled scores over that set (-inf for an empty set).
    Result: L = ln sum_i exp(lse_i) and out = sum_i exp(lse_i - L) out_i; out = 0 and
    L = -inf where every set is empty.
    """
    lse = np.stack([np.asarray(x, np.float64) for x in lses])          # [P, ...]
    o = np.stack([np.asarray(x, np.float64) for x in outs])            # [P, ..., d]
    m = lse.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(lse - m_safe)                                            # exp(-inf) = 0
    s = e.sum(axis=0)
    L = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, s)))
    w = e / np.where(empty, 1.0, s)
    out = (w[..., None] * np.where(np.isneginf(lse)[..., None], 0.0, o)).sum(axis=0)
    return out, L


def cascade_attention(q: np.ndarray, kv_cache: np.ndarray, block_table: np.ndarray,
                      query_start_loc: np.ndarray, seq_lens: np.ndarray, scale: float,
                      causal: bool, common_prefix_len: int) -> Tuple[np.ndarray, np.ndarray]:
    """Prefix pass, suffix pass and merge, as listed in the module docstring.

    Same arguments and results as ``attention`` (window 0), plus ``common_prefix_len``.
    """
    P = int(common_prefix_len)
    bs = kv_cache.shape[2]
    num_tokens = q.shape[0]
    qsl = np.asarray(query_start_loc, np.int64)
    sl = np.asarray(seq_lens, np.int64)
    assert P >= 0 and P % bs == 0
    assert np.all(sl - (qsl[1:] - qsl[:-1]) >= P), "every query must sit after the prefix"
    if P == 0:
        return attention(q, kv_cache, block_table, qsl, sl, scale, causal)
    nb = P // bs
    assert np.all(block_table[:, :nb] == block_table[0, :nb]), "the prefix blocks differ"

    # 1. prefix pass: one sequence, all query tokens, keys = the common prefix, no mask
    o_pre, lse_pre = attention(q, kv_cache, block_table[:1], np.array([0, num_tokens]),
                               np.array([P]), scale, causal=False)
    # 2. suffix pass: each request over its keys after the prefix
    o_suf, lse_suf = attention(q, kv_cache, np.ascontiguousarray(block_table[:, nb:]), qsl,
                               sl - P, scale, causal)
    # 3. merge through the log-sum-exps
    return merge_partials([o_pre, o_suf], [lse_pre, lse_suf])
