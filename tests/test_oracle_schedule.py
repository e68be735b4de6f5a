"""Pins of the work-item oracle (prefill items and their costs from the attention mask):
hand-computed costs for non-causal, causal and windowed tiles, decode rows excluded; each
planted mistake in a copy of the oracle fails one of them."""
import inspect
import types

import pytest

import oracle
import oracle.schedule as osch


def test_non_causal_tiles_read_every_key_tile():
    items = oracle.prefill_items([300, 512], [700, 512], 0, causal=False, window=0)
    assert items == [(0, 0, 11), (0, 1, 11), (1, 0, 8), (1, 1, 8)]


def test_causal_costs_grow_with_the_tile():
    # ql = sl = 1000, no context: tile t sees keys [0, 256 t + 255] (the last tile up to 999)
    items = oracle.prefill_items([1000], [1000], 0, causal=True, window=0)
    assert [c for _, _, c in items] == [4, 8, 12, 16]
    # with a context of 100 keys every tile sees 100 more keys
    items = oracle.prefill_items([1000], [1100], 0, causal=True, window=0)
    assert [c for _, _, c in items] == [(100 + 255) // 64 + 1, (100 + 511) // 64 + 1,
                                        (100 + 767) // 64 + 1, (100 + 999) // 64 + 1]


def test_window_cuts_the_left_edge():
    # W = 100: tile 1 (rows 256..511) sees keys [157, 511] -> tiles 2..7 -> 6
    items = oracle.prefill_items([1000], [1000], 0, causal=True, window=100)
    assert items[1] == (0, 1, 7 - 2 + 1)
    assert items[0] == (0, 0, 255 // 64 + 1)          # rows 0..255 see keys [0, 255]


def test_decode_rows_are_not_items():
    items = oracle.prefill_items([1, 1, 40], [50, 900, 40], 2, causal=True, window=0)
    assert items == [(2, 0, 1)]

MUTATIONS = {
    "cost_counted_from_key_zero": ("int(cols[-1] // tile_keys - cols[0] // tile_keys + 1)",
                                   "int(cols[-1] // tile_keys + 1)"),
    "last_key_tile_not_counted": ("int(cols[-1] // tile_keys - cols[0] // tile_keys + 1)",
                                  "int(cols[-1] // tile_keys - cols[0] // tile_keys)"),
    "decode_rows_included": ("range(num_decodes, len(seq_lens))", "range(0, len(seq_lens))"),
    "tile_rows_overlap": ("vis[t * tile_rows:(t + 1) * tile_rows]",
                          "vis[t * tile_rows:(t + 1) * tile_rows + 1]"),
    "last_partial_tile_dropped": ("range(-(-ql // tile_rows))", "range(ql // tile_rows)"),
}


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_a_planted_schedule_mistake_fails_some_pin(mutation, monkeypatch):
    before, after = MUTATIONS[mutation]
    src = inspect.getsource(osch)
    assert before in src
    src = src.replace("from .naive_attention import", "from oracle.naive_attention import")
    mod = types.ModuleType("oracle_schedule_mutant")
    exec(compile(src.replace(before, after, 1), "oracle_schedule_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(oracle, "prefill_items", mod.prefill_items)
    pins = [test_non_causal_tiles_read_every_key_tile, test_causal_costs_grow_with_the_tile,
            test_window_cuts_the_left_edge, test_decode_rows_are_not_items]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"no pin caught mutation {mutation}"


# ---- decode items: partitions of P keys of the one query row's visible keys
def test_decode_partitions_without_window():
    # keys 0..4999 in 2048-key partitions: 2048, 2048 and 904 keys (57 units of 16, rounded up)
    assert oracle.decode_items([5000], 1, 0, 2048) == [(0, 0, 128), (0, 1, 128), (0, 2, 57)]
    assert oracle.decode_items([4096], 1, 0, 2048) == [(0, 0, 128), (0, 1, 128)]
    assert oracle.decode_items([1, 17], 2, 0, 2048) == [(0, 0, 1), (1, 0, 2)]


def test_decode_window_starts_at_the_first_visible_partition():
    # the row at position 4999 with W = 4096 sees keys [904, 4999]: partition 0 holds 1144 of
    # them (72 units), then 2048 and 904
    assert oracle.decode_items([5000], 1, 4096, 2048) == [(0, 0, 72), (0, 1, 128), (0, 2, 57)]
    # W = 100: keys [4900, 4999], all in partition 2, numbered 0 here
    assert oracle.decode_items([5000], 1, 100, 2048) == [(0, 0, 7)]


def test_decode_items_skip_the_prefix_and_prefill_rows():
    # a pass over the keys after a 2048-key prefix: 2952 keys -> 2048 + 904
    assert oracle.decode_items([5000], 1, 0, 2048, kv_skip=2048) == [(0, 0, 128), (0, 1, 57)]
    assert oracle.decode_items([2048], 1, 0, 2048, kv_skip=2048) == []
    assert oracle.decode_items([30, 900], 1, 0, 512) == [(0, 0, 2)]     # row 1 is prefill


DECODE_MUTATIONS = {
    "partitions_numbered_from_key_zero": ("int(p) - first", "int(p)"),
    "cost_rounded_down": ("int(-(-np.count_nonzero(parts == p) // 16))",
                          "int(np.count_nonzero(parts == p) // 16)"),
    "window_ignored": ("visible_keys(1, sl, True, window)", "visible_keys(1, sl, True, 0)"),
    "prefix_not_skipped": ("int(seq_lens[r]) - kv_skip", "int(seq_lens[r])"),
    "prefill_rows_included": ("for r in range(num_decodes):", "for r in range(len(seq_lens)):"),
}


@pytest.mark.parametrize("mutation", sorted(DECODE_MUTATIONS))
def test_a_planted_decode_schedule_mistake_fails_some_pin(mutation, monkeypatch):
    before, after = DECODE_MUTATIONS[mutation]
    src = inspect.getsource(osch)
    assert before in src
    src = src.replace("from .naive_attention import", "from oracle.naive_attention import")
    mod = types.ModuleType("oracle_schedule_mutant")
    exec(compile(src.replace(before, after, 1), "oracle_schedule_mutant", "exec"), mod.__dict__)
    monkeypatch.setattr(oracle, "decode_items", mod.decode_items)
    pins = [test_decode_partitions_without_window,
            test_decode_window_starts_at_the_first_visible_partition,
            test_decode_items_skip_the_prefix_and_prefill_rows]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"no pin caught mutation {mutation}"
