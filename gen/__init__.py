"""Seeded synthetic inputs for varlen attention over a paged KV cache.

This module holds none of the attention arithmetic. It draws request lengths, builds block
tables over a shuffled block pool, draws N(0,1) query and key/value tensors, and lays them
out in the paged cache format (2, num_blocks, block_size, num_kv_heads, head_size). The
oracle side (tests, the CPU baseline) and the GPU side (tests, bench, smoke) both take their
inputs from here; nothing here imports either side.

Randomness:
  * metadata (lengths, block-pool permutation) comes from numpy's PCG64 seeded with
    ``np.random.SeedSequence([seed, stream])``;
  * tensors come from ``torch.randn`` with a ``torch.Generator`` on the target device,
    seeded from the same SeedSequence scheme, drawn in float32 and rounded to bfloat16
    (round-to-nearest-even) when the workload is bf16. The same seed gives the same bytes on
    the same device type; CPU and GPU streams differ, so a test always hands the oracle the
    very tensors that the GPU path read (copied back to the host).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

# sub-stream ids
_S_LENGTHS, _S_POOL, _S_Q, _S_KV = 1, 2, 3, 4


def _rng(seed: int, stream: int, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, extra])))


def _torch_seed(seed: int, stream: int, extra: int = 0) -> int:
    st = np.random.SeedSequence([seed, stream, extra]).generate_state(2, dtype=np.uint32)
    return int(st[0]) | (int(st[1] & 0x7FFFFFFF) << 32)


@dataclasses.dataclass
class Batch:
    """Host-side metadata of one varlen batch plus its per-layer attention parameters.

    Requests [0, num_decodes) have query_len == 1 and come first (decode-first order).
    ``passes`` lists (causal, window) per layer pass; each pass has its own q and kv tensors.
    """
    name: str
    num_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    dtype: str                      # "bf16" | "f32"
    scale: float
    query_lens: np.ndarray          # int32 [num_seqs]
    seq_lens: np.ndarray            # int32 [num_seqs]
    block_table: np.ndarray         # int32 [num_seqs, max_blocks_per_seq]
    num_blocks: int
    passes: List[Tuple[bool, int]]  # (causal, window) per pass
    pad_block: int                  # block id used for table entries past a request's end
    shared_prefix_blocks: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def query_start_loc(self) -> np.ndarray:
        qsl = np.zeros(self.num_seqs + 1, dtype=np.int32)
        np.cumsum(self.query_lens, out=qsl[1:])
        return qsl

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def num_decodes(self) -> int:
        """Length of the leading run of query_len == 1 requests."""
        n = 0
        for ql in self.query_lens:
            if ql != 1:
                break
            n += 1
        return n

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def blocks_used(self, r: int) -> int:
        return -(-int(self.seq_lens[r]) // self.block_size)


def _build_table(rng: np.random.Generator, seq_lens: np.ndarray, bs: int, pool_factor: int,
                 shared_prefix_blocks: int) -> Tuple[np.ndarray, int, int]:
    """Block table over a randomly permuted pool.

    The first ``shared_prefix_blocks`` entries of every request point to the same physical
    blocks; all other blocks are private. The pool holds pool_factor x the private blocks
    needed plus the shared ones plus one spare block; entries past a request's last block
    point to that spare ("pad") block, which tests fill with NaN.
    """
    nblk = (seq_lens.astype(np.int64) + bs - 1) // bs
    assert np.all(nblk >= shared_prefix_blocks)
    private = int((nblk - shared_prefix_blocks).sum())
    num_blocks = shared_prefix_blocks + private * pool_factor + 1
    perm = rng.permutation(num_blocks).astype(np.int32)
    shared = perm[:shared_prefix_blocks]
    priv = perm[shared_prefix_blocks:shared_prefix_blocks + private]
    pad = int(perm[-1])
    maxb = int(nblk.max()) if nblk.size else 1
    table = np.full((seq_lens.shape[0], maxb), pad, dtype=np.int32)
    pos = 0
    for r, n in enumerate(nblk):
        table[r, :shared_prefix_blocks] = shared
        k = int(n) - shared_prefix_blocks
        table[r, shared_prefix_blocks:int(n)] = priv[pos:pos + k]
        pos += k
    return table, num_blocks, pad


def make_batch(name: str, *, num_heads: int, num_kv_heads: int, head_size: int, block_size: int,
               dtype: str, query_lens: Sequence[int], seq_lens: Sequence[int],
               passes: Sequence[Tuple[bool, int]], seed: int, pool_factor: int = 1,
               shared_prefix_blocks: int = 0, scale: Optional[float] = None) -> Batch:
    ql = np.asarray(query_lens, dtype=np.int32)
    sl = np.asarray(seq_lens, dtype=np.int32)
    assert ql.shape == sl.shape and np.all(sl >= ql) and np.all(ql >= 0)
    table, nb, pad = _build_table(_rng(seed, _S_POOL), sl, block_size, pool_factor,
                                  shared_prefix_blocks)
    return Batch(name=name, num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=head_size,
                 block_size=block_size, dtype=dtype,
                 scale=float(1.0 / math.sqrt(head_size)) if scale is None else float(scale),
                 query_lens=ql, seq_lens=sl, block_table=table, num_blocks=nb,
                 passes=list(passes), pad_block=pad, shared_prefix_blocks=shared_prefix_blocks)


# ----------------------------------------------------------------------------------------
# The five workloads. Lengths "uniform in [a, b]" are inclusive integers.
# ----------------------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny-causal-f32 (1x256, 4 heads, d64, bs256)",
    2: "bert-large-encoder (8x512, 16 heads, d64, non-causal, bs512)",
    3: "gpt2-varlen-causal (16 x U[128,1024], 12 heads, d64, bs16, pool 2x)",
    4: "paged-gqa-decode (256 x U[512,8192], 32q/8kv heads, d128, bs16)",
    5: "mixed-long-context (120 decode U[4096,32768] + 8 prefill q2048, 64q/8kv, d128, bs64, "
       "2048 shared prefix, pass0 causal / pass1 causal W4096)",
}


def config(k: int, seed: Optional[int] = None) -> Batch:
    """Workload k (1..5); seed defaults to k."""
    s = k if seed is None else seed
    rng = _rng(s, _S_LENGTHS)
    if k == 1:
        return make_batch("tiny-causal-f32", num_heads=4, num_kv_heads=4, head_size=64,
                          block_size=256, dtype="f32", query_lens=[256], seq_lens=[256], passes=[(True, 0)],
                          seed=s, scale=1.0 / 8.0)
    if k == 2:
        return make_batch("bert-large-encoder", num_heads=16, num_kv_heads=16, head_size=64,
                          block_size=512, dtype="bf16", query_lens=[512] * 8, seq_lens=[512] * 8,
                          passes=[(False, 0)], seed=s)
    if k == 3:
        sl = rng.integers(128, 1024, size=16, endpoint=True)
        return make_batch("gpt2-varlen-causal", num_heads=12, num_kv_heads=12, head_size=64,
                          block_size=16, dtype="bf16", query_lens=sl, seq_lens=sl, passes=[(True, 0)],
                          seed=s, pool_factor=2)
    if k == 4:
        sl = rng.integers(512, 8192, size=256, endpoint=True)
        return make_batch("paged-gqa-decode", num_heads=32, num_kv_heads=8, head_size=128,
                          block_size=16, dtype="bf16", query_lens=[1] * 256, seq_lens=sl,
                          passes=[(True, 0)], seed=s)
    if k == 5:
        sl_dec = rng.integers(4096, 32768, size=120, endpoint=True)
        sl_pre = rng.integers(4096, 32768, size=8, endpoint=True)
        return make_batch("mixed-long-context", num_heads=64, num_kv_heads=8, head_size=128,
                          block_size=64, dtype="bf16", query_lens=[1] * 120 + [2048] * 8,
                          seq_lens=np.concatenate([sl_dec, sl_pre]),
                          passes=[(True, 0), (True, 4096)], seed=s,
                          shared_prefix_blocks=2048 // 64)
    raise ValueError(f"no workload {k}")


# ----------------------------------------------------------------------------------------
# Tensors
# ----------------------------------------------------------------------------------------
def _torch_dtype(batch: Batch):
    import torch
    return torch.bfloat16 if batch.dtype == "bf16" else torch.float32


def _randn(shape, seed: int, device, dtype, chunk_rows: int = 0):
    """N(0,1) in float32 rounded to ``dtype``; drawn in chunks along dim 0 of ``shape`` when
    chunk_rows > 0 (bounds the float32 temporary for multi-GB caches)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    if chunk_rows <= 0 or shape[0] <= chunk_rows:
        out.copy_(torch.randn(shape, generator=g, device=device, dtype=torch.float32))
        return out
    for a in range(0, shape[0], chunk_rows):
        b = min(shape[0], a + chunk_rows)
        out[a:b].copy_(torch.randn((b - a,) + tuple(shape[1:]), generator=g, device=device,
                                   dtype=torch.float32))
    return out


def make_q(batch: Batch, seed: int, device="cpu", layer: int = 0):
    return _randn((batch.num_tokens, batch.num_heads, batch.head_size),
                  _torch_seed(seed, _S_Q, layer), device, _torch_dtype(batch))


def make_kv(batch: Batch, seed: int, device="cpu", layer: int = 0, poison: bool = False):
    """kv_cache (2, num_blocks, block_size, num_kv_heads, head_size). With ``poison`` every
    slot that no request may read (unused pool blocks, the pad block, and slots at or past
    seq_len in each request's last block) is NaN."""
    import torch
    shape = (2, batch.num_blocks, batch.block_size, batch.num_kv_heads, batch.head_size)
    per_block = batch.block_size * batch.num_kv_heads * batch.head_size
    chunk = max(1, (1 << 26) // per_block)
    kv = torch.empty(shape, dtype=_torch_dtype(batch), device=device)
    for half in range(2):
        kv[half].copy_(_randn(shape[1:], _torch_seed(seed, _S_KV, 2 * layer + half), device,
                              _torch_dtype(batch), chunk_rows=chunk))
    if poison:
        poison_unused(batch, kv)
    return kv


def readable_mask(batch: Batch) -> np.ndarray:
    """bool [num_blocks, block_size]: True where some request's visible range may touch."""
    m = np.zeros((batch.num_blocks, batch.block_size), dtype=bool)
    for r in range(batch.num_seqs):
        sl = int(batch.seq_lens[r])
        for b in range(batch.blocks_used(r)):
            n = min(batch.block_size, sl - b * batch.block_size)
            m[batch.block_table[r, b], :n] = True
    return m


def poison_unused(batch: Batch, kv) -> None:
    import torch
    mask = torch.from_numpy(~readable_mask(batch)).to(kv.device)
    kv[:, mask] = float("nan")


def make_tensors(batch: Batch, seed: int, device="cpu", layer: int = 0, poison: bool = False):
    return make_q(batch, seed, device, layer), make_kv(batch, seed, device, layer, poison)


# ----------------------------------------------------------------------------------------
# Layout helpers used by tests (pure data movement, no arithmetic on values)
# ----------------------------------------------------------------------------------------
def to_numpy_f64(t) -> np.ndarray:
    """Exact upcast of a bf16/f32 torch tensor to a float64 numpy array."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def subset_meta(batch: Batch, requests: Sequence[int]) -> Batch:
    """The same block pool and cache, with the metadata of ``requests`` only (in order)."""
    r = list(requests)
    return dataclasses.replace(batch, name=batch.name + "-requests",
                               query_lens=batch.query_lens[r].copy(),
                               seq_lens=batch.seq_lens[r].copy(),
                               block_table=batch.block_table[r].copy())


def subset(batch: Batch, requests: Sequence[int], q, kv):
    """A smaller batch holding only ``requests`` (in the given order), with its own compact
    block pool and remapped table; returns (sub_batch, q_sub, kv_sub) as host torch tensors.
    Shared blocks stay shared. Used to hand large workloads to the oracle piecewise."""
    import torch
    requests = list(requests)
    qsl = batch.query_start_loc
    blocks: List[int] = []
    remap = {}
    for r in requests:
        for b in range(batch.blocks_used(r)):
            pb = int(batch.block_table[r, b])
            if pb not in remap:
                remap[pb] = len(blocks)
                blocks.append(pb)
    maxb = max(batch.blocks_used(r) for r in requests)
    table = np.zeros((len(requests), maxb), dtype=np.int32)
    for i, r in enumerate(requests):
        for b in range(batch.blocks_used(r)):
            table[i, b] = remap[int(batch.block_table[r, b])]
    sub = dataclasses.replace(
        batch, name=batch.name + "-subset", query_lens=batch.query_lens[requests].copy(),
        seq_lens=batch.seq_lens[requests].copy(), block_table=table, num_blocks=len(blocks),
        pad_block=0)
    idx = torch.as_tensor(blocks, dtype=torch.long, device=kv.device)
    kv_sub = kv.index_select(1, idx).cpu()
    rows = np.concatenate([np.arange(qsl[r], qsl[r + 1]) for r in requests]) if requests else []
    q_sub = q.index_select(0, torch.as_tensor(rows, dtype=torch.long, device=q.device)).cpu()
    return sub, q_sub, kv_sub


def contiguous_twin(batch: Batch, kv):
    """The same batch with one block per request (block_size = max_seq_len rounded up to 16),
    request r in block r: the 'one KV block per request' layout."""
    import torch
    bs = max(16, -(-batch.max_seq_len // 16) * 16)
    S = batch.num_seqs
    out = torch.zeros((2, S, bs, batch.num_kv_heads, batch.head_size), dtype=kv.dtype,
                      device=kv.device)
    for r in range(S):
        sl = int(batch.seq_lens[r])
        for t0 in range(0, sl, batch.block_size):
            n = min(batch.block_size, sl - t0)
            out[:, r, t0:t0 + n] = kv[:, int(batch.block_table[r, t0 // batch.block_size]), :n]
    twin = dataclasses.replace(batch, name=batch.name + "-contig", block_size=bs,
                               block_table=np.arange(S, dtype=np.int32).reshape(S, 1),
                               num_blocks=S, pad_block=0, shared_prefix_blocks=0)
    return twin, out
