"""Pins for the oracle's block/slot arithmetic and pool scatter/gather (CPU only)."""

import itertools

import numpy as np

from oracle import paging


def test_block_size_4_example(golden):
    g = golden("paging_block_size_4.json")
    bs, bt = g["block_size"], g["block_table"]
    assert paging.blocks_needed(g["seq_len"], bs) == g["blocks_for_10_tokens"]
    for lk in g["lookups"]:
        assert paging.locate(lk["pos"], bs) == (lk["logical_block"], lk["offset"])
        assert paging.slot_of(bt, lk["pos"], bs) == lk["physical_block"] * bs + lk["offset"]
    for ap in g["appends"]:
        assert paging.slot_of(bt, ap["pos"], bs) == ap["physical_block"] * bs + ap["offset"]
    assert paging.slot_mapping(bt, 10, 2, bs) == [78, 79]
    p = g["first_pos_needing_new_block"]
    assert paging.locate(p, bs)[0] == len(bt)          # beyond the 3-entry table
    assert paging.locate(p - 1, bs)[0] == len(bt) - 1


def test_block_rounding(golden):
    g = golden("block_rounding.json")
    n = paging.blocks_needed(g["tokens"], g["block_size"])
    assert n == g["blocks"]
    assert n * g["block_size"] == g["slots"]
    assert paging.tail_waste(g["tokens"], g["block_size"]) == g["empty_slots"]
    # the 36th token (position 35) lands in the third block, offset 3: no new block
    assert paging.locate(35, 16) == (2, 3)
    assert paging.blocks_needed(36, 16) == 3


def test_scatter_gather_all_tables_of_a_tiny_pool():
    """Brute force: every ordered choice of blocks from a 4-block pool, every length."""
    bs, hkv, dh = 2, 2, 3
    rng = np.random.default_rng(0)
    for n_used in range(1, 5):
        for table in itertools.permutations(range(4), n_used):
            for t in range((n_used - 1) * bs + 1, n_used * bs + 1):
                kv = rng.normal(size=(t, hkv, dh)).astype(np.float32)
                pool = np.full((4, hkv, bs, dh), np.nan, dtype=np.float32)
                paging.scatter(pool, kv, list(table), bs)
                back = paging.gather(pool, list(table), t, bs)
                assert np.array_equal(back, np.transpose(kv, (1, 0, 2)))
                # exactly t slots written, the rest keep the sentinel
                written = ~np.isnan(pool[:, 0, :, 0])
                assert written.sum() == t
                slots = paging.slot_mapping(list(table), 0, t, bs)
                assert len(set(slots)) == t
                for s, p in zip(slots, range(t)):
                    assert np.array_equal(pool[s // bs, :, s % bs, :], kv[p])


def test_append_skips_minus_one_and_matches_scatter():
    bs = 4
    table = [7, 2, 19]
    kv = np.arange(12 * 1 * 2, dtype=np.float32).reshape(12, 1, 2)
    a = np.full((20, 1, bs, 2), np.nan, dtype=np.float32)
    paging.scatter(a, kv, table, bs)
    b = np.full((20, 1, bs, 2), np.nan, dtype=np.float32)
    slots = paging.slot_mapping(table, 0, 12, bs)
    paging.append(b, kv, slots, bs)
    assert np.array_equal(a, b, equal_nan=True)
    c = np.full((20, 1, bs, 2), np.nan, dtype=np.float32)
    paging.append(c, kv, [-1 if i % 3 == 0 else s for i, s in enumerate(slots)], bs)
    assert np.isnan(c).sum() == np.isnan(b).sum() + 4 * 2


def test_logical_order_survives_relabelling():
    """Paging changes storage, not order: two different tables gather the same sequence."""
    rng = np.random.default_rng(1)
    bs, t = 4, 13
    kv = rng.normal(size=(t, 1, 5))
    p1 = np.full((8, 1, bs, 5), np.nan)
    p2 = np.full((8, 1, bs, 5), np.nan)
    paging.scatter(p1, kv, [0, 1, 2, 3], bs)
    paging.scatter(p2, kv, [6, 3, 7, 1], bs)
    assert np.array_equal(paging.gather(p1, [0, 1, 2, 3], t, bs), paging.gather(p2, [6, 3, 7, 1], t, bs))
    assert not np.array_equal(p1, p2, equal_nan=True)
