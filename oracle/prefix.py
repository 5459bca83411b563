"""Exact-prefix reuse over full blocks, with chained block keys.

Pages:
* "04. 注意力与 KV 缓存", section on sharing a prefix across requests and its
  explicit-token demo: cached ABCDEFGHIJKL vs new ABCDEFGXIJKL share 7 tokens;
  only whole pages are reusable, 4 tokens here (so the page holds 4 tokens),
  and at least 8 must be recomputed; after the first difference nothing can be
  reused even where later tokens agree again.
* same page, engine section: the full-block key chains the parent block's key,
  this block's tokens and extra identity (model, adapter, …).
* "06 KV Cache…", section 6.4: full cached blocks are keyed by a chained hash of
  the parent key and the block's tokens; whether a partial block is reusable is
  an implementation detail (read here: it is not); 6.4 also defines the token
  hit rate as hit tokens / comparable prompt tokens and the request hit rate as
  requests with any hit / requests.

Keys here are nested tuples, so two keys are equal exactly when the whole chain
of tokens and identity is equal — the property a hashed key approximates.
"""


def common_prefix(a, b):
    n = 0
    for x, y in zip(a, b):
        if x != y:
            break
        n += 1
    return n


def reusable_tokens(cached, new, page):
    """Tokens whose cached state can be reused: the common prefix rounded down
    to whole pages."""
    return (common_prefix(cached, new) // page) * page


def block_keys(tokens, page, identity=()):
    """Chained keys of the full blocks of `tokens` (a trailing partial block has none)."""
    keys = []
    parent = ("root", tuple(identity))
    for i in range(len(tokens) // page):
        parent = (parent, tuple(tokens[i * page:(i + 1) * page]))
        keys.append(parent)
    return keys


class PrefixIndex:
    """Maps chained full-block keys to physical block ids."""

    def __init__(self, page):
        self.page = page
        self.table = {}
        self.hit_tokens = 0
        self.compared_tokens = 0
        self.requests = 0
        self.hit_requests = 0

    def insert(self, tokens, block_ids, identity=()):
        for key, bid in zip(block_keys(tokens, self.page, identity), block_ids):
            self.table.setdefault(key, bid)

    def match(self, tokens, identity=()):
        """Physical ids of the longest chain of cached full blocks; stops at the
        first miss. Updates the hit counters."""
        ids = []
        for key in block_keys(tokens, self.page, identity):
            bid = self.table.get(key)
            if bid is None:
                break
            ids.append(bid)
        self.requests += 1
        self.hit_requests += 1 if ids else 0
        self.compared_tokens += len(tokens)
        self.hit_tokens += len(ids) * self.page
        return ids
