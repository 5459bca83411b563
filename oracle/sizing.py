"""KV-cache byte arithmetic.

Page "07｜…内部过程", Q026 (how much memory the cache takes) and its unit table:
KV bytes = 2 × L × B × T × H_kv × Dh × bytes-per-element, the leading 2 being K
and V; with L = 32, B = 1, T = 32768, H_kv = 8, Dh = 128 at 2 bytes that is
4 GiB, 128 KiB per extra token, 16 GiB with 32 KV heads.
Page "06 KV Cache…", section 6.3: the same formula, ΣT_i replacing B·T for
varied lengths; N = 32, T = 8192, H_kv = 8, d = 128, bf16 gives 1 GiB.
Page "07｜…内部过程", chapter warm-up check: one layer, 3 positions, 4 numbers a
row gives 24 numbers for K and V together.
"""


def kv_elements(layers, batch, tokens, kv_heads, head_dim):
    """Numbers stored for K and V together."""
    return 2 * layers * batch * tokens * kv_heads * head_dim


def kv_bytes(layers, batch, tokens, kv_heads, head_dim, bytes_per_element):
    return kv_elements(layers, batch, tokens, kv_heads, head_dim) * bytes_per_element


def kv_bytes_varlen(layers, seq_lens, kv_heads, head_dim, bytes_per_element):
    """ΣT_i in place of B·T."""
    return 2 * layers * sum(int(t) for t in seq_lens) * kv_heads * head_dim * bytes_per_element


def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_element):
    return kv_bytes(layers, 1, 1, kv_heads, head_dim, bytes_per_element)
