"""Pins of the cache-write oracle (slot_mapping scatter).

The pins fix the write against facts that do not come from the oracle: a hand-placed
example, the read path of the attention oracle (a token written to slot s must be what
gather_kv reads back for the position the block table maps to s), untouched slots, padding
slots, and the layer step (write the new tokens, then attend) matching attention over a cache
built directly. Planted mistakes in the write must fail one of them."""
import inspect
import types

import numpy as np
import pytest

import gen
import oracle
import oracle.kv_write as okw


def test_hand_placed_example():
    kv = np.zeros((2, 3, 4, 2, 2))
    key = np.arange(8, dtype=np.float64).reshape(2, 2, 2)
    val = -key
    out = oracle.kv_cache_write(kv, key, val, np.array([9, 2]))   # block 2 slot 1, block 0 slot 2
    exp = np.zeros_like(kv)
    exp[0, 2, 1] = key[0]; exp[1, 2, 1] = val[0]
    exp[0, 0, 2] = key[1]; exp[1, 0, 2] = val[1]
    np.testing.assert_array_equal(out, exp)
    assert not np.shares_memory(out, kv) and not kv.any()


def test_padding_slots_are_skipped_and_other_slots_untouched():
    rng = np.random.default_rng(0)
    kv = rng.normal(size=(2, 5, 16, 3, 8))
    key, val = rng.normal(size=(4, 3, 8)), rng.normal(size=(4, 3, 8))
    slots = np.array([-1, 17, -5, 79])
    out = oracle.kv_cache_write(kv, key, val, slots)
    touched = np.zeros((5, 16), bool)
    touched[1, 1] = touched[4, 15] = True
    np.testing.assert_array_equal(out[:, ~touched], kv[:, ~touched])
    np.testing.assert_array_equal(out[0, 1, 1], key[1])
    np.testing.assert_array_equal(out[1, 4, 15], val[3])


@pytest.mark.parametrize("bs", [16, 32])
def test_written_tokens_are_what_the_read_path_gathers(bs):
    # appending the last ql tokens of each request through slot_mapping and reading the
    # request back through its block table gives the appended rows at positions cl .. sl-1
    b = gen.make_batch("kvw", num_heads=4, num_kv_heads=2, head_size=8, block_size=bs,
                       dtype="f32", query_lens=[5, 1, 40], seq_lens=[30, 77, 40],
                       passes=[(True, 0)], seed=3, pool_factor=2)
    rng = np.random.default_rng(bs)
    kv = rng.normal(size=(2, b.num_blocks, bs, 2, 8))
    qsl = b.query_start_loc
    key, val = rng.normal(size=(b.num_tokens, 2, 8)), rng.normal(size=(b.num_tokens, 2, 8))
    slots = np.empty(b.num_tokens, np.int64)
    for r in range(b.num_seqs):
        cl = int(b.seq_lens[r] - b.query_lens[r])
        for i in range(int(b.query_lens[r])):
            p = cl + i
            slots[qsl[r] + i] = int(b.block_table[r, p // bs]) * bs + p % bs
    out = oracle.kv_cache_write(kv, key, val, slots)
    for r in range(b.num_seqs):
        k, v = oracle.gather_kv(out, b.block_table[r], int(b.seq_lens[r]))
        cl = int(b.seq_lens[r] - b.query_lens[r])
        np.testing.assert_array_equal(k[cl:], key[qsl[r]:qsl[r + 1]])
        np.testing.assert_array_equal(v[cl:], val[qsl[r]:qsl[r + 1]])
        k0, v0 = oracle.gather_kv(kv, b.block_table[r], cl)
        np.testing.assert_array_equal(k[:cl], k0)                  # the context is kept
        np.testing.assert_array_equal(v[:cl], v0)


MUTATIONS = {
    "k_and_v_swapped": ("out[0, blk, off] = key[t]", "out[0, blk, off] = value[t]"),
    "block_offset_transposed": ("blk, off = divmod(int(slot), block_size)",
                                "off, blk = divmod(int(slot), block_size)"),
    "padding_not_skipped": ("if slot < 0:", "if slot < -10**9:"),
    "off_by_one_token": ("out[1, blk, off] = value[t]", "out[1, blk, off] = value[t - 1]"),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_a_planted_write_mistake_fails_some_pin(mutation, monkeypatch):
    before, after = MUTATIONS[mutation]
    src = inspect.getsource(okw)
    assert before in src
    mod = types.ModuleType("oracle_kv_write_mutant")
    exec(compile(src.replace(before, after, 1), "oracle_kv_write_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(oracle, "kv_cache_write", mod.kv_cache_write)
    pins = [test_hand_placed_example, test_padding_slots_are_skipped_and_other_slots_untouched,
            lambda: test_written_tokens_are_what_the_read_path_gathers(16)]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"no pin caught mutation {mutation}"
