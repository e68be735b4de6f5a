"""Plain fp64 "naive attention" over a paged KV cache, written out from its definition.

Test infrastructure: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg
use this module.

What it computes (sources are the pages this project follows):
  * RBLN "Attention 모드" page, section 개요 (Overview), the "Naive Attention" bullet:
    attention scores over the valid tokens, a softmax over them, and the weights times V.
  * vLLM FlashAttention page ("[vLLM] FlashAttention: IO-aware 타일링으로 ..."), section
    들어가며 (Intro): Q.K^T, softmax, then multiplication by V. Its "왜 이 설계인가" item 4
    states that the tiled method is exact, so the plain definition is the oracle.
  * Same page, "FlashAttentionBackend" section: the cache shape
    (2, num_blocks, block_size, num_kv_heads, head_size); index 0 of the first axis is K,
    index 1 is V. "FlashAttentionMetadata" section: query_start_loc, seq_lens, block_table.
  * Same page, "FlashAttentionImpl" section: ``scale`` is a parameter and
    num_queries_per_kv = num_heads // num_kv_heads (GQA).
  * vLLM other-backends page ("[vLLM] 기타 Attention Backends ..."), section
    "Triton Attention": context_len = tokens before this step, query_len = new tokens,
    seq_len = context_len + query_len.
  * RBLN page, "Full Attention" (causal masking) and "Sliding-Window Attention(SWA)"
    (only tokens inside the window).

Readings where the pages are silent (all also listed in the design notes):
  * query i of a request sits at absolute position p = context_len + i and, when causal,
    sees keys j <= p (bottom-right alignment);
  * a window W > 0 keeps keys j >= p - W + 1, i.e. W keys including the query's own;
  * q head h reads kv head h // (num_heads // num_kv_heads);
  * lse is the natural-log log-sum-exp of the scaled scores over the visible keys;
  * a row with no visible key has out = 0 and lse = -inf.

Every value is upcast to float64 before any arithmetic.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def gather_kv(kv_cache: np.ndarray, table_row: np.ndarray, seq_len: int
              ) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of one request as float64 [seq_len, num_kv_heads, head_size].

    Logical token t lives in physical block table_row[t // block_size] at slot
    t % block_size (the paged layout of the FlashAttentionBackend section)."""
    block_size = kv_cache.shape[2]
    t = np.arange(seq_len)
    blocks = np.asarray(table_row)[t // block_size]
    slots = t % block_size
    k = np.asarray(kv_cache[0][blocks, slots], dtype=np.float64)
    v = np.asarray(kv_cache[1][blocks, slots], dtype=np.float64)
    return k, v


def visible_keys(query_len: int, seq_len: int, causal: bool, window: int) -> np.ndarray:
    """bool [query_len, seq_len]: entry (i, j) says whether query i may attend to key j."""
    context_len = seq_len - query_len
    p = context_len + np.arange(query_len)[:, None]     # absolute position of query i
    j = np.arange(seq_len)[None, :]
    vis = np.ones((query_len, seq_len), dtype=bool)
    if causal:
        vis &= j <= p
    if window > 0:
        vis &= j >= p - window + 1
    return vis


def softmax_weights(scores: np.ndarray, vis: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Row-wise softmax of ``scores`` restricted to ``vis``; returns (weights, lse).

    weights are 0 on invisible keys; a row with no visible key gets all-zero weights and
    lse = -inf."""
    s = np.where(vis, scores, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(vis, np.exp(s - m_safe), 0.0)
    l = e.sum(axis=1, keepdims=True)
    w = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return w, lse[:, 0]


def attend_rows(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                vis: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One head: q_rows [n, d], k and v [seq_len, d], vis [n, seq_len] -> (out [n, d], lse [n])."""
    scores = scale * (np.asarray(q_rows, np.float64) @ np.asarray(k, np.float64).T)
    w, lse = softmax_weights(scores, vis)
    return w @ np.asarray(v, np.float64), lse


def attention(q: np.ndarray, kv_cache: np.ndarray, block_table: np.ndarray,
              query_start_loc: np.ndarray, seq_lens: np.ndarray, scale: float, causal: bool,
              window: int = 0, rows: Optional[Sequence[int]] = None, row_chunk: int = 256
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention for a varlen batch.

    q         [num_tokens, num_heads, head_size]   (any float dtype; upcast to float64)
    kv_cache  [2, num_blocks, block_size, num_kv_heads, head_size]
    returns   out float64 [num_tokens, num_heads, head_size], lse float64 [num_tokens, num_heads]

    ``rows`` restricts the work to the listed token indices; other rows are NaN. Rows are
    independent by definition, so they are processed in chunks: for each kv head, the
    (query, q head) rows of its GQA group go through attend_rows together, at most
    ``row_chunk`` of them at a time (each row's scores, softmax and x V are its own; sharing
    one product only saves re-reading that kv head's keys per q head).
    """
    num_tokens, num_heads, head_size = q.shape
    num_kv_heads = kv_cache.shape[3]
    assert num_heads % num_kv_heads == 0
    group = num_heads // num_kv_heads
    out = np.full((num_tokens, num_heads, head_size), np.nan)
    lse = np.full((num_tokens, num_heads), np.nan)
    want = None
    if rows is not None:
        want = np.zeros(num_tokens, dtype=bool)
        want[np.asarray(rows, dtype=np.int64)] = True
    for r in range(len(seq_lens)):
        q0, q1 = int(query_start_loc[r]), int(query_start_loc[r + 1])
        ql, sl = q1 - q0, int(seq_lens[r])
        idx = np.arange(ql)
        if want is not None:
            idx = idx[want[q0:q1]]
        if idx.size == 0:
            continue
        k, v = gather_kv(kv_cache, block_table[r], sl)
        vis_all = visible_keys(ql, sl, causal, window)
        step = max(1, row_chunk // group)
        for kvh in range(num_kv_heads):
            heads = np.arange(kvh * group, (kvh + 1) * group)   # q head h reads kv head h // group
            k_h = np.ascontiguousarray(k[:, kvh])
            v_h = np.ascontiguousarray(v[:, kvh])
            for c0 in range(0, idx.size, step):
                ii = idx[c0:c0 + step]
                # rows (query i, q head h) of this group, query-major
                q_rows = q[q0 + ii][:, heads].reshape(ii.size * group, head_size)
                vis = np.repeat(vis_all[ii], group, axis=0)
                o, ls = attend_rows(q_rows, k_h, v_h, scale, vis)
                out[np.ix_(q0 + ii, heads)] = o.reshape(ii.size, group, head_size)
                lse[np.ix_(q0 + ii, heads)] = ls.reshape(ii.size, group)
    return out, lse


def flops_visible_pairs(query_lens: Sequence[int], seq_lens: Sequence[int], causal: bool,
                        window: int) -> int:
    """Number of visible (query, key) pairs of a batch, per head (counted, not computed on
    a matrix, so it also works at full size)."""
    total = 0
    for ql, sl in zip(query_lens, seq_lens):
        ql, sl = int(ql), int(sl)
        cl = sl - ql
        p = cl + np.arange(ql, dtype=np.int64)
        hi = np.minimum(p + 1, sl) if causal else np.full(ql, sl, dtype=np.int64)
        lo = np.maximum(p - window + 1, 0) if window > 0 else np.zeros(ql, dtype=np.int64)
        total += int(np.maximum(hi - lo, 0).sum())
    return total
