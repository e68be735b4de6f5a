"""Pins of the work-item oracle (prefill items and their costs from the attention mask):
hand-computed costs for non-causal, causal and windowed tiles, decode rows excluded."""
import numpy as np

import oracle


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
