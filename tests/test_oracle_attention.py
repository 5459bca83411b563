"""Pins for the oracle's attention definition (CPU only).

The oracle materialises softmax(QKᵀ·scale + inclusive causal mask)·V. It is
pinned against torch's scaled_dot_product_attention in float64 (a library
routine written independently), closed-form special cases and structured probes.
"""

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention


def _rand(rng, *shape):
    return rng.normal(size=shape)


def _sdpa(q, k, v, scale, causal):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(torch.float64)  # noqa: E731
    return F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale).numpy()


@pytest.mark.parametrize("t,dh", [(1, 8), (7, 16), (33, 64)])
def test_full_causal_matches_sdpa(t, dh):
    rng = np.random.default_rng(t)
    h = 3
    q, k, v = _rand(rng, h, t, dh), _rand(rng, h, t, dh), _rand(rng, h, t, dh)
    scale = 1 / np.sqrt(dh)
    ours = attention.causal_attention(q, k, v, np.arange(t), scale)
    assert np.allclose(ours, _sdpa(q, k, v, scale, True), atol=1e-12)


def test_decode_matches_unmasked_sdpa():
    rng = np.random.default_rng(1)
    b, hq, dh = 3, 4, 32
    lens = [1, 17, 40]
    q = _rand(rng, b, hq, dh)
    ks = [_rand(rng, hq, t, dh) for t in lens]
    vs = [_rand(rng, hq, t, dh) for t in lens]
    out = attention.decode(q, ks, vs, 0.25)
    for i in range(b):
        want = _sdpa(q[i][:, None, :], ks[i], vs[i], 0.25, False)[:, 0, :]
        assert np.allclose(out[i], want, atol=1e-12)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(2)
    hq, hkv, t, dh = 8, 2, 21, 16
    q, k, v = _rand(rng, hq, 5, dh), _rand(rng, hkv, t, dh), _rand(rng, hkv, t, dh)
    pos = np.arange(t - 5, t)
    ours = attention.causal_attention(q, k, v, pos, 0.3)
    rep = lambda a: np.repeat(a, hq // hkv, axis=0)  # noqa: E731  contiguous groups
    mha = attention.causal_attention(q, rep(k), rep(v), pos, 0.3)
    assert np.array_equal(ours, mha)
    # and the same through the library routine (last 5 rows of a full causal pass)
    qfull = np.concatenate([_rand(rng, hq, t - 5, dh), q], axis=1)
    want = _sdpa(qfull, rep(k), rep(v), 0.3, True)[:, -5:, :]
    assert np.allclose(ours, want, atol=1e-12)


def test_mqa_single_kv_head():
    rng = np.random.default_rng(3)
    q, k, v = _rand(rng, 6, 1, 8), _rand(rng, 1, 9, 8), _rand(rng, 1, 9, 8)
    ours = attention.causal_attention(q, k, v, [8], 0.5)
    for h in range(6):
        want = _sdpa(q[h:h + 1], k, v, 0.5, False)
        assert np.allclose(ours[h], want[0], atol=1e-12)


def test_chunk_is_tail_of_full_causal_and_decode_is_chunk_of_one():
    rng = np.random.default_rng(4)
    hq, hkv, p, c, dh = 4, 2, 13, 6, 16
    t = p + c
    qall = _rand(rng, t, hq, dh)
    k, v = _rand(rng, hkv, t, dh), _rand(rng, hkv, t, dh)
    chunk = attention.prefill_chunk(qall[p:], k, v, 0.2)
    full = attention.prefill_chunk(qall, k, v, 0.2)        # P = 0: the whole sequence
    assert np.allclose(chunk, full[p:], atol=1e-13)
    rep = lambda a: np.repeat(a, hq // hkv, axis=0)  # noqa: E731
    want = _sdpa(np.transpose(qall, (1, 0, 2)), rep(k), rep(v), 0.2, True)
    assert np.allclose(full, np.transpose(want, (1, 0, 2)), atol=1e-12)
    # decode of the last token == a chunk of one
    dec = attention.decode(qall[-1][None], [k], [v], 0.2)[0]
    assert np.allclose(dec, chunk[-1], atol=1e-14)


def test_single_key_returns_its_value_exactly():
    rng = np.random.default_rng(5)
    q, k, v = _rand(rng, 2, 1, 8), _rand(rng, 2, 1, 8), _rand(rng, 2, 1, 8)
    assert np.array_equal(attention.causal_attention(q, k, v, [0], 1.0), v)


def test_zero_query_gives_mean_of_visible_rows():
    rng = np.random.default_rng(6)
    t = 11
    k, v = _rand(rng, 1, t, 4), _rand(rng, 1, t, 4)
    q = np.zeros((1, t, 4))
    out = attention.causal_attention(q, k, v, np.arange(t), 1.0)
    for i in range(t):
        assert np.allclose(out[0, i], v[0, :i + 1].mean(axis=0), atol=1e-14)


def test_position_probe():
    """q = 0 and V[t] = t/T in dim 0: the output is (T-1)/(2T); a dropped or
    duplicated token moves it."""
    for t in (1, 2, 36, 100):
        k = np.random.default_rng(t).normal(size=(1, t, 8))
        v = np.zeros((1, t, 8))
        v[0, :, 0] = np.arange(t) / t
        out = attention.decode(np.zeros((1, 1, 8)), [k], [v], 0.125)
        assert out[0, 0, 0] == pytest.approx((t - 1) / (2 * t), abs=1e-14)


def test_peaked_probe():
    rng = np.random.default_rng(8)
    t, dh = 50, 16
    k, v = _rand(rng, 1, t, dh), _rand(rng, 1, t, dh)
    q = k[0, 17] * 40.0
    out = attention.decode(q[None, None, :], [k], [v], 1 / np.sqrt(dh))
    assert np.allclose(out[0, 0], v[0, 17], atol=1e-6)


def test_empty_sequence_gives_zeros():
    out = attention.decode(np.ones((2, 2, 4)), [np.zeros((1, 0, 4)), np.ones((1, 3, 4))],
                           [np.zeros((1, 0, 4)), np.ones((1, 3, 4))], 1.0)
    assert np.array_equal(out[0], np.zeros((2, 4)))
    assert np.allclose(out[1], 1.0)


def test_planted_exclusive_mask_is_caught():
    """An exclusive diagonal (j < p) is a plausible mistake; the sdpa pin catches it."""
    rng = np.random.default_rng(9)
    q, k, v = _rand(rng, 1, 6, 8), _rand(rng, 1, 6, 8), _rand(rng, 1, 6, 8)
    want = _sdpa(q, k, v, 0.3, True)
    orig = attention.causal_attention
    def wrong(q, k, v, q_pos, scale):
        return orig(q, k, v, np.asarray(q_pos) - 1 + (np.asarray(q_pos) == 0), scale)
    assert not np.allclose(wrong(q, k, v, np.arange(6), 0.3), want, atol=1e-6)


def test_planted_interleaved_grouping_is_caught():
    """Grouping h % Hkv instead of h // G breaks the repeated-heads pin."""
    rng = np.random.default_rng(10)
    hq, hkv, t, dh = 4, 2, 9, 8
    q, k, v = _rand(rng, hq, 1, dh), _rand(rng, hkv, t, dh), _rand(rng, hkv, t, dh)
    rep = np.repeat(k, 2, axis=0), np.repeat(v, 2, axis=0)
    want = _sdpa(q, rep[0], rep[1], 0.4, False)
    wrong_k = np.stack([k[h % hkv] for h in range(hq)])
    wrong_v = np.stack([v[h % hkv] for h in range(hq)])
    got = attention.causal_attention(q, k, v, [t - 1], 0.4)
    assert np.allclose(got, want, atol=1e-12)
    assert not np.allclose(_sdpa(q, wrong_k, wrong_v, 0.4, False), want, atol=1e-6)
