"""Pins for the allocator model, KV byte arithmetic and prefix reuse (CPU only)."""

import numpy as np
import pytest

from oracle import allocator, prefix, sizing
from oracle.allocator import EINVAL, ENOBLOCKS, EREF, OK


# ---- sizing -----------------------------------------------------------------

def test_kv_bytes_page_values(golden):
    g = golden("kv_bytes.json")
    for c in g["cases"]:
        got = sizing.kv_bytes(c["layers"], c["batch"], c["tokens"], c["kv_heads"], c["head_dim"], c["bytes"])
        assert got == c["kv_bytes"], c["cite"]
        if "k_elements" in c:
            assert sizing.kv_elements(c["layers"], c["batch"], c["tokens"], c["kv_heads"], c["head_dim"]) // 2 == c["k_elements"]
            assert got // 2 == c["k_bytes"]
    pt = g["per_token"]
    assert sizing.kv_bytes_per_token(pt["layers"], pt["kv_heads"], pt["head_dim"], pt["bytes"]) == pt["value"]
    cc = g["count_check"]
    assert sizing.kv_elements(cc["layers"], 1, cc["positions"], 1, cc["numbers_per_row"]) == cc["k_and_v_numbers"]
    assert sizing.kv_bytes_varlen(32, [8192] * 8, 8, 128, 2) == 8 * 2 ** 30


# ---- allocator model ----------------------------------------------------------

def _invariants(a):
    live = sum(1 for r in a.ref if r > 0)
    assert live + a.num_free() == a.num_blocks
    assert len(set(a.free)) == len(a.free)
    assert all(a.ref[i] == 0 for i in a.free)


def test_page_example_growth():
    """bs 4: 10 tokens in 3 blocks; positions 10, 11 need no block; 12 does."""
    a = allocator.ModelAllocator(32, 4)
    st, t, cow = a.reserve_append([-1] * 8, 0, 10)
    assert st == OK and cow == [] and sum(1 for x in t if x >= 0) == 3
    free_before = a.num_free()
    st, t2, cow = a.reserve_append(t, 10, 2)
    assert st == OK and t2 == t and a.num_free() == free_before
    st, t3, cow = a.reserve_append(t2, 12, 1)
    assert st == OK and a.num_free() == free_before - 1 and t3[3] >= 0 and t3[:3] == t2[:3]
    _invariants(a)


def test_35_then_36():
    a = allocator.ModelAllocator(8, 16)
    st, t, _ = a.reserve_append([-1] * 3, 0, 35)
    assert st == OK and a.num_free() == 5
    st, t2, _ = a.reserve_append(t, 35, 1)
    assert st == OK and t2 == t and a.num_free() == 5


def test_shared_partial_tail_copies_on_write_and_full_blocks_do_not():
    a = allocator.ModelAllocator(16, 4)
    st, ta, _ = a.reserve_append([-1] * 4, 0, 6)        # blocks: full + half
    assert st == OK
    assert a.incref(ta[:2]) == OK                        # B shares both
    tb = list(ta)
    st, ta2, cow = a.reserve_append(ta, 6, 1)           # A writes into the shared tail
    assert st == OK and len(cow) == 1 and cow[0][0] == ta[1] and ta2[1] == cow[0][1]
    assert a.refcount(ta[1]) == 1 and a.refcount(ta2[1]) == 1 and a.refcount(ta[0]) == 2
    st, tb2, cow = a.reserve_append(tb, 6, 1)           # B is now sole owner: no copy
    assert st == OK and cow == [] and tb2 == tb
    # a shared *full* block is never copied
    a2 = allocator.ModelAllocator(16, 4)
    st, t, _ = a2.reserve_append([-1] * 4, 0, 8)
    a2.incref(t[:2])
    st, t2, cow = a2.reserve_append(t, 8, 3)
    assert st == OK and cow == [] and t2[:2] == t[:2]
    _invariants(a)
    _invariants(a2)


def test_errors_leave_state_unchanged():
    a = allocator.ModelAllocator(4, 4)
    st, t, _ = a.reserve_append([-1] * 8, 0, 12)
    snap = (list(a.ref), list(a.free))
    assert a.reserve_append(t, 12, 8)[0] == ENOBLOCKS    # needs 2, has 1
    assert (list(a.ref), list(a.free)) == snap
    assert a.allocate(2)[0] == ENOBLOCKS
    assert a.decref([t[0], t[0]]) == EREF                 # refcount 1, two decrefs
    assert (list(a.ref), list(a.free)) == snap
    assert a.incref([a.free[-1]]) == EREF                 # not live
    assert a.incref([99]) == EINVAL
    assert a.reserve_append(t, 12, 40)[0] == EINVAL       # beyond max_blocks
    assert (list(a.ref), list(a.free)) == snap


def test_free_only_at_zero():
    a = allocator.ModelAllocator(4, 4, free_order=[3, 1, 0, 2])
    st, ids = a.allocate(1)
    assert ids == [3]
    a.incref(ids)
    a.decref(ids)
    assert a.num_free() == 3 and 3 not in a.free
    a.decref(ids)
    assert a.num_free() == 4 and a.free[-1] == 3         # LIFO: next allocation reuses it
    assert a.allocate(1)[1] == [3]


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(3)
    a = allocator.ModelAllocator(40, 4)
    seqs = []                                            # [table, seq_len]
    for _ in range(2000):
        op = int(rng.integers(0, 4))
        if op == 0 or not seqs:
            n = int(rng.integers(0, 20))
            st, t, _ = a.reserve_append([-1] * 10, 0, n)
            if st == OK:
                seqs.append([t, n])
        elif op == 1:
            i = int(rng.integers(len(seqs)))
            t, n = seqs[i]
            k = int(rng.integers(0, 6))
            st, t2, cow = a.reserve_append(t, n, k)
            if st == OK:
                assert len(cow) <= 1
                seqs[i] = [t2, n + k]
        elif op == 2:
            i = int(rng.integers(len(seqs)))
            t, n = seqs[i]
            live = [x for x in t if x >= 0]
            if a.incref(live) == OK:
                seqs.append([list(t), n])
        else:
            i = int(rng.integers(len(seqs)))
            t, _ = seqs.pop(i)
            assert a.decref([x for x in t if x >= 0]) == OK
        _invariants(a)
        # every live table entry is referenced at least as often as tables hold it
        held = {}
        for t, _ in seqs:
            for x in t:
                if x >= 0:
                    held[x] = held.get(x, 0) + 1
        assert all(a.ref[x] == c for x, c in held.items())
    for t, _ in seqs:
        assert a.decref([x for x in t if x >= 0]) == OK
    assert a.num_free() == 40


# ---- prefix reuse -------------------------------------------------------------

def test_prefix_demo(golden):
    g = golden("prefix_demo.json")
    cached, new = list(g["cached"]), list(g["new"])
    assert prefix.common_prefix(cached, new) == g["common_prefix"]
    pages = [p for p in range(2, 13) if prefix.reusable_tokens(cached, new, p) == g["reusable_full_page_tokens"]]
    assert pages == [4]
    reuse = prefix.reusable_tokens(cached, new, 4)
    assert len(new) - reuse == g["min_recomputed"]


def test_prefix_index_stops_at_first_miss_and_counts_hits():
    idx = prefix.PrefixIndex(4)
    idx.insert(list("ABCDEFGHIJKL"), [10, 11, 12])
    assert idx.match(list("ABCDEFGXIJKL")) == [10]
    assert idx.match(list("XBCDEFGHIJKL")) == []          # edit at the start: nothing reusable
    assert idx.match(list("ABCDEFGHIJKLMN")) == [10, 11, 12]
    assert idx.match(list("ABCDEFGHIJKL"), identity=("other-adapter",)) == []
    assert idx.requests == 4 and idx.hit_requests == 2
    assert idx.hit_tokens == 4 + 12 and idx.compared_tokens == 12 + 12 + 14 + 12
    # the same block of tokens after a different parent is a different key
    idx.insert(list("ZZZZEFGH"), [20, 21])
    assert idx.match(list("ABCDEFGH")) == [10, 11]


# ---- positions whose K/V are built during generation -------------------------

def _brute_force_positions(prompt, generated, cached):
    """Simulate the steps with a set standing in for the cache: a step's
    forward pass covers positions 0 … prompt + k − 1; each one whose K/V is not
    held is built (and, with a cache, kept)."""
    held, built = set(), []
    for k in range(generated):
        n = 0
        for pos in range(prompt + k):
            if pos not in held:
                n += 1
                if cached:
                    held.add(pos)
        built.append(n)
    return built


def test_positions_built_page_values(golden):
    g = golden("positions_built.json")
    r = g["long_request"]
    without = sizing.positions_built_per_step(r["prompt"], r["generated"], cached=False)
    assert without[0] == r["first_step"] and without[1] == r["second_step_without_cache"]
    assert without[-1] == r["last_step_without_cache"]
    assert sum(without) == r["without_cache"]
    assert sizing.positions_built(r["prompt"], r["generated"], cached=True) == r["with_cache"]
    ratio = r["without_cache"] / r["with_cache"]
    assert abs(ratio - r["ratio_printed_about"]) < 0.02 * r["ratio_printed_about"]   # 171.5
    t = g["three_rounds"]
    per = sizing.positions_built_per_step(t["prompt"], t["generated"], cached=True)
    assert per == t["with_cache_per_round"] and sum(per) == t["with_cache_total"]


@pytest.mark.parametrize("prompt,generated", [(1, 1), (1, 5), (4, 3), (7, 9), (30, 12)])
def test_positions_built_brute_force(prompt, generated):
    for cached in (False, True):
        assert sizing.positions_built_per_step(prompt, generated, cached) == \
            _brute_force_positions(prompt, generated, cached)
    # quadratic against linear growth: the gap widens with the output length
    assert sizing.positions_built(prompt, generated, False) >= sizing.positions_built(prompt, generated, True)
