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


# ---- positions whose K/V are built during generation ------------------------
# Page "03. KV Cache：用显存换计算", section on how much is recomputed without a
# cache: without a cache every step feeds the whole history through the model
# again, so step k builds K/V for the prompt plus the k − 1 tokens generated so
# far; with a cache the first step (prefill) builds the prompt's K/V and every
# later step builds only the one new position. Its table of three rounds counts
# 4, then 1, then 1 new positions with the cache.

def positions_built_per_step(prompt_tokens, generated_tokens, cached):
    """K/V positions built at each of the generated_tokens steps."""
    steps = []
    have = 0                      # positions whose K/V survive from earlier steps
    for k in range(generated_tokens):
        seen = prompt_tokens + k  # history the step-k forward pass attends over
        if cached:
            steps.append(seen - have)
            have = seen
        else:
            steps.append(seen)
    return steps


def positions_built(prompt_tokens, generated_tokens, cached):
    return sum(positions_built_per_step(prompt_tokens, generated_tokens, cached))
