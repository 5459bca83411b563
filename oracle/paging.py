"""Block tables, slots and the paged pool, by plain loops.

Page "07｜…内部过程", Q028 (PagedAttention): a sequence's logically contiguous
KV is cut into fixed-size blocks mapped to a pool of physical blocks; the worked
table with block size 4 and table [7, 2, 19] locates logical position 5 at
logical block 5 // 4 = 1, offset 5 % 4 = 1, i.e. physical block 2 offset 1;
positions 10 and 11 fill block 19 at offsets 2 and 3; position 12 is the first
that needs a fourth block. Paging changes where tokens live, not their logical
order (closing line of that table).

Page "06 KV Cache…", section 6.5: 35 tokens at block size 16 need 3 blocks,
48 slots, 13 of them empty at the tail.

Pool layout used by the library and mirrored here: [num_blocks, Hkv, bs, Dh];
the flat slot of a token is physical_block * bs + offset.
"""

import numpy as np


def blocks_needed(num_tokens, block_size):
    """ceil(T / bs) blocks for T tokens."""
    return -(-int(num_tokens) // int(block_size))


def tail_waste(num_tokens, block_size):
    """Empty slots in the last block: blocks·bs − T."""
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


def locate(pos, block_size):
    """Logical position → (logical block, offset within block)."""
    return pos // block_size, pos % block_size


def slot_of(block_table, pos, block_size):
    """Logical position → flat slot via the sequence's block table."""
    lb, off = locate(pos, block_size)
    return int(block_table[lb]) * block_size + off


def slot_mapping(block_table, first_pos, n, block_size):
    """Slots for n consecutive new tokens starting at logical position first_pos."""
    return [slot_of(block_table, first_pos + i, block_size) for i in range(n)]


def scatter(pool, kv, block_table, block_size, first_pos=0):
    """Write a sequence's tokens into the pool, one token at a time.

    pool: [num_blocks, Hkv, bs, Dh] (modified in place)
    kv:   [N, Hkv, Dh] tokens at logical positions first_pos … first_pos + N − 1
    """
    for i in range(kv.shape[0]):
        s = slot_of(block_table, first_pos + i, block_size)
        pool[s // block_size, :, s % block_size, :] = kv[i]
    return pool


def append(pool, kv_new, slots, block_size):
    """The append step with an explicit slot mapping; slot −1 means skip.

    Reading for the skip value: the pages are silent; −1 marks padding tokens.
    """
    for i, s in enumerate(slots):
        s = int(s)
        if s < 0:
            continue
        pool[s // block_size, :, s % block_size, :] = kv_new[i]
    return pool


def gather(pool, block_table, num_tokens, block_size):
    """Read a sequence back into the semantic layout [Hkv, T, Dh]."""
    nb, hkv, bs, dh = pool.shape
    assert bs == block_size
    out = np.empty((hkv, num_tokens, dh), dtype=pool.dtype)
    for p in range(num_tokens):
        s = slot_of(block_table, p, block_size)
        out[:, p, :] = pool[s // block_size, :, s % block_size, :]
    return out
