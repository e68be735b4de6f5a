"""The seeded generator: determinism, the workload recipes, and the paged pool structure."""
import numpy as np
import pytest
import torch

import gen


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_metadata_is_deterministic_and_in_range(k):
    a, b = gen.config(k), gen.config(k)
    assert np.array_equal(a.seq_lens, b.seq_lens) and np.array_equal(a.block_table, b.block_table)
    c = gen.config(k, seed=1000 + k)
    if k in (3, 4, 5):
        assert not np.array_equal(a.seq_lens, c.seq_lens)
    assert np.all(a.seq_lens >= a.query_lens)
    assert a.block_size % 16 == 0
    # every block a request uses is a valid, distinct physical block (shared prefix aside)
    used = []
    for r in range(a.num_seqs):
        n = a.blocks_used(r)
        row = a.block_table[r, :n]
        assert np.all((row >= 0) & (row < a.num_blocks))
        used.extend(row[a.shared_prefix_blocks:].tolist())
        assert np.all(a.block_table[r, n:] == a.pad_block)
    assert len(used) == len(set(used)) and a.pad_block not in used


def test_workload_shapes():
    c3 = gen.config(3)
    assert c3.num_seqs == 16 and c3.seq_lens.min() >= 128 and c3.seq_lens.max() <= 1024
    assert np.array_equal(c3.seq_lens, c3.query_lens) and c3.num_decodes == 0
    need = sum(c3.blocks_used(r) for r in range(16))
    assert c3.num_blocks == 2 * need + 1
    c4 = gen.config(4)
    assert c4.num_decodes == 256 and c4.seq_lens.min() >= 512 and c4.seq_lens.max() <= 8192
    assert (c4.num_heads, c4.num_kv_heads, c4.head_size, c4.block_size) == (32, 8, 128, 16)
    c5 = gen.config(5)
    assert c5.num_decodes == 120 and c5.num_tokens == 120 + 8 * 2048
    assert c5.passes == [(True, 0), (True, 4096)]
    assert np.all(c5.seq_lens >= 4096) and np.all(c5.seq_lens <= 32768)
    shared = c5.block_table[:, :32]
    assert np.all(shared == shared[0])                     # one 2048-token prefix for all
    c1 = gen.config(1)
    assert c1.dtype == "f32" and c1.scale == 1.0 / 8.0 and c1.block_size == 256


def test_tensors_deterministic_and_bf16_rounded():
    b = gen.make_batch("t", num_heads=4, num_kv_heads=2, head_size=64, block_size=16,
                       dtype="bf16", query_lens=[5, 9], seq_lens=[20, 9], passes=[(True, 0)],
                       seed=9, pool_factor=2)
    q1, kv1 = gen.make_tensors(b, 9)
    q2, kv2 = gen.make_tensors(b, 9)
    assert torch.equal(q1, q2) and torch.equal(kv1, kv2)
    assert q1.dtype == torch.bfloat16 and kv1.shape == (2, b.num_blocks, 16, 2, 64)
    q3, _ = gen.make_tensors(b, 10)
    assert not torch.equal(q1, q3)
    x = q1.float()
    assert abs(x.mean().item()) < 0.1 and abs(x.std().item() - 1) < 0.1


def test_poison_marks_exactly_the_unreadable_slots():
    b = gen.make_batch("t", num_heads=2, num_kv_heads=1, head_size=64, block_size=16,
                       dtype="bf16", query_lens=[3, 1], seq_lens=[37, 16], passes=[(True, 0)],
                       seed=4, pool_factor=2)
    kv = gen.make_kv(b, 4, poison=True)
    nan = torch.isnan(kv[0, :, :, 0, 0]).numpy()
    readable = gen.readable_mask(b)
    assert np.array_equal(nan, ~readable)
    assert readable.sum() == 37 + 16


def test_subset_and_contiguous_twin_move_data_only():
    b = gen.make_batch("t", num_heads=2, num_kv_heads=1, head_size=8, block_size=16,
                       dtype="f32", query_lens=[3, 1, 4], seq_lens=[37, 16, 40],
                       passes=[(True, 0)], seed=5, pool_factor=2, )
    q, kv = gen.make_tensors(b, 5)
    sub, qs, kvs = gen.subset(b, [2, 0], q, kv)
    qsl = b.query_start_loc
    assert torch.equal(qs, torch.cat([q[qsl[2]:qsl[3]], q[qsl[0]:qsl[1]]]))
    for i, r in enumerate([2, 0]):
        for t in range(int(b.seq_lens[r])):
            a = kv[:, b.block_table[r, t // 16], t % 16]
            c = kvs[:, sub.block_table[i, t // 16], t % 16]
            assert torch.equal(a, c)
    twin, kvc = gen.contiguous_twin(b, kv)
    for r in range(3):
        for t in range(int(b.seq_lens[r])):
            assert torch.equal(kvc[:, r, t], kv[:, b.block_table[r, t // 16], t % 16])
