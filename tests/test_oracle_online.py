"""Pins for the oracle's online-softmax state and merge (CPU only)."""

import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import online


def two_block_pin_holds(mod, golden):
    """True when `mod` reproduces the page's two-block table to its printed digits."""
    g = golden("online_softmax_two_blocks.json")
    b1, b2 = g["blocks"]
    st = mod.update(mod.empty(1), b1["scores"], b1["values"])
    ok = (st.m == g["after_block_1"]["m"] and st.l == g["after_block_1"]["l"]
          and np.allclose(st.u, g["after_block_1"]["u"], atol=0, rtol=0))
    st = mod.update(st, b2["scores"], b2["values"])
    tol = 0.5 * 10.0 ** -g["printed_decimals"]
    want = g["after_block_2"]
    ok = ok and st.m == want["m"]
    ok = ok and abs(st.l - want["l"]) <= tol
    ok = ok and abs(st.u[0] - want["u"][0]) <= tol
    ok = ok and abs(mod.finish(st)[0] - want["o"][0]) <= tol
    return bool(ok)


def test_two_block_example_matches_page(golden):
    assert two_block_pin_holds(online, golden)


def test_two_block_closed_form():
    st = online.run_blocks([1.0, 3.0], [[2.0], [10.0]], [1, 1])
    e = math.e
    assert st.l == pytest.approx(math.exp(-2) + 1, abs=1e-15)
    assert st.u[0] == pytest.approx(2 * math.exp(-2) + 10, abs=1e-14)
    assert online.finish(st)[0] == pytest.approx((2 * e + 10 * e ** 3) / (e + e ** 3), abs=1e-13)


class _NoRescale:
    """The page's wrong variant: the maximum moves but old l and u are not scaled."""
    empty = staticmethod(online.empty)
    finish = staticmethod(online.finish)

    @staticmethod
    def update(state, scores, values):
        s = np.asarray(scores, dtype=np.float64)
        v = np.asarray(values, dtype=np.float64).reshape(len(s), -1)
        m_new = max(state.m, s.max())
        w = np.exp(s - m_new)
        if not np.isfinite(state.m):
            return online.State(m_new, w.sum(), w @ v)
        return online.State(m_new, state.l + w.sum(), state.u + w @ v)


class _OnlyLRescaled(_NoRescale):
    @staticmethod
    def update(state, scores, values):
        s = np.asarray(scores, dtype=np.float64)
        v = np.asarray(values, dtype=np.float64).reshape(len(s), -1)
        m_new = max(state.m, s.max())
        w = np.exp(s - m_new)
        if not np.isfinite(state.m):
            return online.State(m_new, w.sum(), w @ v)
        a = np.exp(state.m - m_new)
        return online.State(m_new, a * state.l + w.sum(), state.u + w @ v)


@pytest.mark.parametrize("variant,expected_wrong", [(_NoRescale, 6.0), (_OnlyLRescaled, 10.5696)])
def test_pin_rejects_missing_rescale(golden, variant, expected_wrong):
    """A merge that forgets α must fail the page pin (planted mistakes)."""
    st = variant.update(variant.update(online.empty(1), [1.0], [[2.0]]), [3.0], [[10.0]])
    assert online.finish(st)[0] == pytest.approx(expected_wrong, abs=1e-4)
    assert not two_block_pin_holds(variant, golden)


def _three_key_closed_form():
    w = np.array([1.0, math.exp(2.0), math.exp(1.0)])
    v = np.array([[5.0, 5.0], [10.0, 0.0], [0.0, 20.0]])
    return (w @ v) / w.sum()


def test_single_query_three_keys_states_and_output(golden):
    g = golden("single_query_three_keys.json")
    s, v = g["scores"], g["values"]
    st = online.update(online.empty(2), s[:1], v[:1])
    assert (st.m, st.l) == (0.0, 1.0) and np.array_equal(st.u, [5.0, 5.0])
    st = online.update(st, s[1:2], v[1:2])
    assert st.m == 2.0
    assert st.l == pytest.approx(1.135335283, abs=1e-9)
    assert np.allclose(st.u, [10.676676416, 0.676676416], atol=1e-9)
    st = online.update(st, s[2:3], v[2:3])
    assert st.m == 2.0
    assert st.l == pytest.approx(1.503214724, abs=1e-9)
    assert np.allclose(st.u, [10.676676416, 8.034265240], atol=1e-9)
    o = online.finish(st)
    assert np.allclose(o, [7.102562424, 5.344722287], atol=1e-9)
    assert np.allclose(o, _three_key_closed_form(), atol=1e-13)
    # a library routine gives the same weights
    assert np.allclose(o, softmax(np.array(s)) @ np.array(v), atol=1e-13)


def test_read_order_and_split_independence(golden):
    g = golden("single_query_three_keys.json")
    s = np.array(g["scores"])
    v = np.array(g["values"])
    ref = _three_key_closed_form()
    for perm in itertools.permutations(range(3)):
        p = list(perm)
        for sizes in ([1, 1, 1], [2, 1], [1, 2], [3]):
            st = online.run_blocks(s[p], v[p], sizes)
            assert np.allclose(online.finish(st), ref, atol=1e-12)


def test_merge_of_partials_equals_full_softmax():
    rng = np.random.default_rng(7)
    for _ in range(50):
        n = int(rng.integers(1, 40))
        s = rng.normal(size=n) * 4
        v = rng.normal(size=(n, 5))
        cuts = sorted(rng.choice(np.arange(1, n), size=min(n - 1, int(rng.integers(0, 4))), replace=False)) if n > 1 else []
        bounds = [0] + list(cuts) + [n]
        parts = [online.from_block(s[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        st = parts[0]
        for p in parts[1:]:
            st = online.merge(st, p)
        assert np.allclose(online.finish(st), softmax(s) @ v, atol=1e-12)
        assert st.m == s.max()


def test_merge_with_empty_partial_is_identity():
    a = online.from_block([0.5, -1.0], [[1.0, 2.0], [3.0, 4.0]])
    m = online.merge(a, online.empty(2))
    assert m.m == a.m and m.l == a.l and np.array_equal(m.u, a.u)
    m = online.merge(online.empty(2), a)
    assert m.m == a.m and m.l == a.l and np.array_equal(m.u, a.u)
