"""Materialised causal attention in float64 — the definition the library must reach.

Pages:
* "04. 注意力与 KV 缓存", section 深入：注意力公式与缓存成立条件 (the attention
  formula) and "03. KV Cache：用显存换计算", section 注意力的公式: attention is
  softmax(Q·Kᵀ/√d + causal mask)·V with d the per-head width.
* "07｜…内部过程", Q025 table row 2: a position sees itself and every earlier
  position (inclusive causal mask); Q025 core answer: the semantic cache layout
  is K and V each [B, H_kv, T, Dh].
* "06 KV Cache…", section 6.3: GQA keeps every query head's scores; query
  heads share KV heads. The grouping is not stated; this oracle reads it as
  contiguous groups, query head h uses KV head h // (Hq / Hkv).

Nothing here knows about blocks or tables: K and V arrive contiguous.
"""

import numpy as np


def causal_attention(q, k, v, q_pos, scale):
    """softmax(q·Kᵀ·scale + causal mask)·V for one sequence, fully materialised.

    q:      [Hq, Nq, Dh]  queries (any real dtype; promoted to float64)
    k, v:   [Hkv, T, Dh]  the sequence's cached keys/values, logical order
    q_pos:  [Nq]          logical position of each query; key j is visible to
                          query i iff j <= q_pos[i] (self included)
    scale:  the score scale (1/sqrt(Dh) in every workload)
    returns [Hq, Nq, Dh] float64
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    hq, nq, dh = q.shape
    hkv, t, dh2 = k.shape
    assert dh == dh2 and v.shape == k.shape and hq % hkv == 0
    group = hq // hkv
    out = np.zeros((hq, nq, dh), dtype=np.float64)
    if t == 0 or nq == 0:
        return out
    visible = np.arange(t)[None, :] <= q_pos[:, None]          # [Nq, T]
    for h in range(hq):
        g = h // group
        s = (q[h] @ k[g].T) * scale                            # [Nq, T]
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1, keepdims=True)                       # row max (identity)
        p = np.exp(s - m)
        p = p / p.sum(axis=1, keepdims=True)
        out[h] = p @ v[g]
    return out


def decode(q, ks, vs, scale):
    """One decode step for a batch: each sequence's single new query sits at the
    last cached position T_b - 1 (its own K/V already appended, page 07 Q025
    "generate a new token" paragraph; page 06 section 6.1), so it sees all T_b keys.

    q:      [B, Hq, Dh]
    ks, vs: length-B lists of [Hkv, T_b, Dh]
    returns [B, Hq, Dh] float64; a sequence with T_b = 0 yields zeros (reading
    for an empty cache: nothing to attend to).
    """
    q = np.asarray(q, dtype=np.float64)
    b, hq, dh = q.shape
    out = np.zeros((b, hq, dh), dtype=np.float64)
    for i in range(b):
        t = ks[i].shape[1]
        if t == 0:
            continue
        out[i] = causal_attention(q[i][:, None, :], ks[i], vs[i], [t - 1], scale)[:, 0, :]
    return out


def prefill_chunk(q, k, v, scale):
    """A causal chunk of C queries on top of a cached prefix of P tokens.

    The chunk's own K/V are already in k, v (total length P + C); query i sits at
    position P + i and sees keys 0 … P + i (page 06 section 6.6 names chunked
    prefill; the visibility rule is the causal mask above).

    q: [C, Hq, Dh]; k, v: [Hkv, P + C, Dh]; returns [C, Hq, Dh] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    c = q.shape[0]
    t = k.shape[1]
    p0 = t - c
    assert p0 >= 0
    o = causal_attention(np.transpose(q, (1, 0, 2)), k, v, np.arange(p0, t), scale)
    return np.transpose(o, (1, 0, 2))
