"""Online softmax state and block merge, in float64.

Page "07｜…内部过程", Q027 (推导在线softmax合并, the online-softmax merge):
for one query keep the running maximum m, the exponent sum l = Σ exp(s_j − m)
and the unnormalised weighted sum u = Σ exp(s_j − m)·v_j; the output is u / l.
When a new block with maximum m_b arrives, m_new = max(m_old, m_b), the old
statistics are multiplied by α = exp(m_old − m_new), and the new block's terms
are added with exponents taken against m_new. Forgetting α gives a wrong result
(the page's worked two-block table, last row).

The split-KV reduce combines several finished partial states the same way: each
partial is rescaled by exp(m_part − m_total) before l and u are summed.
"""

import numpy as np


class State:
    """(m, l, u) for one query row; u has the value width."""

    __slots__ = ("m", "l", "u")

    def __init__(self, m, l, u):
        self.m = float(m)
        self.l = float(l)
        self.u = np.asarray(u, dtype=np.float64)


def empty(width):
    """The state before any block: no maximum yet, zero sums."""
    return State(-np.inf, 0.0, np.zeros(width, dtype=np.float64))


def from_block(scores, values):
    """State of a single block of scores s_j and value rows v_j."""
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    v = np.asarray(values, dtype=np.float64).reshape(len(s), -1)
    m = s.max()
    w = np.exp(s - m)
    return State(m, w.sum(), w @ v)


def update(state, scores, values):
    """Fold one new block of raw scores into a running state (page order)."""
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    v = np.asarray(values, dtype=np.float64).reshape(len(s), -1)
    m_new = max(state.m, s.max())
    alpha = np.exp(state.m - m_new) if np.isfinite(state.m) else 0.0
    w = np.exp(s - m_new)
    return State(m_new, alpha * state.l + w.sum(), alpha * state.u + w @ v)


def merge(a, b):
    """Combine two finished partial states (the split-KV reduce)."""
    m = max(a.m, b.m)
    if not np.isfinite(m):
        return State(m, 0.0, a.u * 0.0)
    wa = np.exp(a.m - m) if np.isfinite(a.m) else 0.0
    wb = np.exp(b.m - m) if np.isfinite(b.m) else 0.0
    return State(m, wa * a.l + wb * b.l, wa * a.u + wb * b.u)


def finish(state):
    """o = u / l."""
    return state.u / state.l


def run_blocks(scores, values, block_sizes):
    """Stream scores/values through `update` in consecutive blocks of the given sizes."""
    s = np.asarray(scores, dtype=np.float64).reshape(-1)
    v = np.asarray(values, dtype=np.float64).reshape(len(s), -1)
    assert sum(block_sizes) == len(s)
    st = empty(v.shape[1])
    i = 0
    for n in block_sizes:
        st = update(st, s[i:i + n], v[i:i + n])
        i += n
    return st
