"""A pure-Python model of the ref-counted block allocator.

Pages:
* "07｜…内部过程", Q028 core answer and its follow-ups: blocks are handed out on
  demand as a sequence grows and go back to the pool when released; sequences
  with an identical prefix may share its blocks with a reference count, and
  writing into a shared, partly filled last block needs copy-on-write, or one
  sequence's append would corrupt the other's (table row 6).
* "06 KV Cache…", section 6.5: allocate on demand → map position to block and
  offset → grow by blocks → release or keep; shared prefix blocks are read-only
  with reference counts and copy-on-write.
* "04. 注意力与 KV 缓存", section on how engines find state: a request that ends
  must not free pages another request still uses.

Readings where the pages are silent (the block numbers there are hypothetical):
* the free pool is a LIFO stack; by default pops return 0, 1, 2, …, or the
  order given by `free_order`;
* every call is all-or-nothing: on error the state is unchanged;
* only a shared, partially filled tail block is copied on write; full shared
  blocks are never written by an append, so they stay shared.

Status codes mirror the library's: 0 ok, -1 invalid argument, -2 out of
blocks, -4 reference-count misuse.
"""

OK, EINVAL, ENOBLOCKS, EREF = 0, -1, -2, -4


class ModelAllocator:
    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if free_order is None else [int(i) for i in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of 0..num_blocks-1")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.ref = [0] * num_blocks
        self.free = list(reversed(order))          # stack: pop() yields order[0] first

    # ---- basic operations -------------------------------------------------
    def num_free(self):
        return len(self.free)

    def refcount(self, bid):
        if not 0 <= bid < self.num_blocks:
            return EINVAL
        return self.ref[bid]

    def allocate(self, n):
        if n < 0:
            return EINVAL, []
        if n > len(self.free):
            return ENOBLOCKS, []
        ids = [self.free.pop() for _ in range(n)]
        for i in ids:
            self.ref[i] = 1
        return OK, ids

    def incref(self, ids):
        for i in ids:
            if not 0 <= i < self.num_blocks:
                return EINVAL
        for i in ids:
            if self.ref[i] <= 0:
                return EREF
        for i in ids:
            self.ref[i] += 1
        return OK

    def decref(self, ids):
        for i in ids:
            if not 0 <= i < self.num_blocks:
                return EINVAL
        need = {}
        for i in ids:
            need[i] = need.get(i, 0) + 1
        for i, c in need.items():
            if self.ref[i] < c:
                return EREF
        for i in ids:
            self.ref[i] -= 1
            if self.ref[i] == 0:
                self.free.append(i)
        return OK

    # ---- growth with copy-on-write -----------------------------------------
    def reserve_append(self, table, seq_len, n_new):
        """Make `table` cover positions [seq_len, seq_len + n_new).

        `table` is a Python list of physical ids (its length is the table's
        capacity, max_blocks; unused entries are -1). Returns
        (status, new_table, cow_pairs) where cow_pairs lists (src, dst) copies
        the caller must perform before writing.
        """
        bs = self.block_size
        max_blocks = len(table)
        if seq_len < 0 or n_new < 0:
            return EINVAL, table, []
        have = -(-seq_len // bs)
        need_total = -(-(seq_len + n_new) // bs)
        if need_total > max_blocks:
            return EINVAL, table, []
        for lb in range(have):
            if not 0 <= table[lb] < self.num_blocks or self.ref[table[lb]] <= 0:
                return EINVAL, table, []
        cow = n_new > 0 and seq_len % bs != 0 and self.ref[table[have - 1]] > 1
        fresh = need_total - have
        if fresh + (1 if cow else 0) > len(self.free):
            return ENOBLOCKS, table, []
        new_table = list(table)
        pairs = []
        if cow:
            src = new_table[have - 1]
            _, (dst,) = self.allocate(1)
            self.ref[src] -= 1                      # > 0 still: it was shared
            new_table[have - 1] = dst
            pairs.append((src, dst))
        if fresh:
            _, ids = self.allocate(fresh)
            new_table[have:need_total] = ids
        return OK, new_table, pairs
