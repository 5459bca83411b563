// Prefix-cache index over full KV blocks (host side).
//
// "04. 注意力与 KV 缓存", section on sharing a prompt prefix and its token demo:
// requests that share a prefix can reuse its cached K/V, but only in whole
// pages and only up to the first token that differs (later agreement does not
// count). Same page, engine section: the key of a full block chains its
// parent's key, its own tokens and extra identity (model, adapter, …).
// "06 KV Cache、Prefix Cache、PagedAttention 与 vLLM" 6.4: full blocks are
// keyed by a chained hash of the parent and the block's tokens, a partial
// block is not reused (the reading taken here), the token hit rate is hit
// tokens over compared prompt tokens and the request hit rate is requests
// with any hit over requests.
//
// Each entry stores its parent entry, identity and tokens, so a lookup
// compares them exactly: the 64-bit chained hash only picks the candidates,
// and two keys match exactly when their whole chains of tokens and identity
// are equal. Bound to an allocator, an indexed block holds one reference
// (released by pkv_prefix_clear) and a match hands the caller one reference
// per matched block.
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "errors.h"

namespace {

struct Entry {
  int32_t parent;      // entry index, −1 at the root
  int32_t block;       // physical block holding this block's K/V
  int32_t next;        // next entry with the same hash, −1 at the end
  bool holds_ref;      // the index holds an allocator reference on `block`
  uint64_t identity;
  uint64_t hash;
};

// splitmix64's output function (Steele, Lea and Flood; constants as
// published for SplittableRandom / splitmix64).
inline uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

inline uint64_t root_hash(uint64_t identity) { return mix64(identity ^ 0x6a09e667f3bcc909ull); }

inline uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int32_t page) {
  uint64_t h = parent;
  for (int32_t i = 0; i < page; ++i) h = mix64(h + 0x9e3779b97f4a7c15ull + (uint32_t)tokens[i]);
  return h;
}

}  // namespace

struct pkv_prefix {
  int32_t page;
  std::vector<Entry> entries;
  std::vector<int32_t> tokens;                    // `page` tokens per entry
  std::unordered_map<uint64_t, int32_t> head;     // hash → first entry with it
  int64_t hit_tokens = 0, compared_tokens = 0, requests = 0, hit_requests = 0;

  // the entry for block `tok` under `parent` (hash `h`), or −1
  int32_t find(int32_t parent, uint64_t identity, uint64_t h, const int32_t* tok) const {
    const auto it = head.find(h);
    for (int32_t e = it == head.end() ? -1 : it->second; e >= 0; e = entries[e].next) {
      const Entry& x = entries[e];
      if (x.parent == parent && x.identity == identity &&
          std::memcmp(&tokens[(size_t)e * page], tok, sizeof(int32_t) * page) == 0)
        return e;
    }
    return -1;
  }

  // Walks the chain of full blocks of tok[0..n): entries of the matched
  // blocks go to `matched` (up to `limit`); returns the parent entry and hash
  // at the first block not matched.
  void walk(const int32_t* tok, int32_t nblk, uint64_t identity, int32_t limit, std::vector<int32_t>& matched,
            int32_t* parent_out, uint64_t* hash_out) const {
    int32_t parent = -1;
    uint64_t h = root_hash(identity);
    matched.clear();
    for (int32_t i = 0; i < nblk && (int32_t)matched.size() < limit; ++i) {
      const uint64_t hi = chain_hash(h, tok + (size_t)i * page, page);
      const int32_t e = find(parent, identity, hi, tok + (size_t)i * page);
      if (e < 0) break;
      matched.push_back(e);
      parent = e;
      h = hi;
    }
    *parent_out = parent;
    *hash_out = h;
  }
};

extern "C" {

PKV_API int pkv_prefix_create(int32_t block_size, pkv_prefix** out) {
  pkv::clear_error();
  if (!out) return pkv::fail(PKV_EINVAL, "pkv_prefix_create: out is NULL");
  *out = nullptr;
  if (block_size <= 0) return pkv::fail(PKV_EINVAL, "pkv_prefix_create: block_size must be positive");
  pkv_prefix* p = new (std::nothrow) pkv_prefix;
  if (!p) return pkv::fail(PKV_EINVAL, "pkv_prefix_create: out of host memory");
  p->page = block_size;
  *out = p;
  return PKV_OK;
}

PKV_API void pkv_prefix_destroy(pkv_prefix* p) { delete p; }

PKV_API int pkv_prefix_insert(pkv_prefix* p, pkv_alloc* alloc, const int32_t* tokens, int32_t n_tokens,
                              uint64_t identity, const int32_t* block_ids, int32_t n_block_ids, int32_t* n_new) {
  pkv::clear_error();
  if (n_new) *n_new = 0;
  if (!p || n_tokens < 0 || n_block_ids < 0 || (n_tokens > 0 && !tokens) || (n_block_ids > 0 && !block_ids))
    return pkv::fail(PKV_EINVAL, "pkv_prefix_insert: bad argument");
  const int32_t nblk = std::min(n_tokens / p->page, n_block_ids);
  std::vector<int32_t> matched;
  int32_t parent;
  uint64_t h;
  p->walk(tokens, nblk, identity, nblk, matched, &parent, &h);
  const int32_t first_new = (int32_t)matched.size();     // every later block is new too
  const int32_t count = nblk - first_new;
  if (count == 0) return PKV_OK;
  if (alloc) {   // the index takes a reference on each newly indexed block
    if (int st = pkv_alloc_incref(alloc, block_ids + first_new, count)) return st;
  } else {
    for (int32_t i = first_new; i < nblk; ++i)
      if (block_ids[i] < 0) return pkv::fail(PKV_EINVAL, "pkv_prefix_insert: negative block id");
  }
  p->entries.reserve(p->entries.size() + count);
  p->tokens.reserve(p->tokens.size() + (size_t)count * p->page);
  for (int32_t i = first_new; i < nblk; ++i) {
    const int32_t* tok = tokens + (size_t)i * p->page;
    const uint64_t hi = chain_hash(h, tok, p->page);
    const int32_t e = (int32_t)p->entries.size();
    auto it = p->head.find(hi);
    const int32_t next = it == p->head.end() ? -1 : it->second;
    p->entries.push_back(Entry{parent, block_ids[i], next, alloc != nullptr, identity, hi});
    p->tokens.insert(p->tokens.end(), tok, tok + p->page);
    p->head[hi] = e;
    parent = e;
    h = hi;
  }
  if (n_new) *n_new = count;
  return PKV_OK;
}

PKV_API int pkv_prefix_match(pkv_prefix* p, pkv_alloc* alloc, const int32_t* tokens, int32_t n_tokens,
                             uint64_t identity, int32_t* out_ids, int32_t max_ids, int32_t* n_match) {
  pkv::clear_error();
  if (!p || !n_match || n_tokens < 0 || max_ids < 0 || (n_tokens > 0 && !tokens) || (max_ids > 0 && !out_ids))
    return pkv::fail(PKV_EINVAL, "pkv_prefix_match: bad argument");
  *n_match = 0;
  std::vector<int32_t> matched;
  int32_t parent;
  uint64_t h;
  p->walk(tokens, n_tokens / p->page, identity, max_ids, matched, &parent, &h);
  const int32_t n = (int32_t)matched.size();
  for (int32_t i = 0; i < n; ++i) out_ids[i] = p->entries[matched[i]].block;
  if (alloc && n > 0) {   // the caller now shares the matched blocks
    if (int st = pkv_alloc_incref(alloc, out_ids, n)) return st;
  }
  p->requests += 1;
  p->hit_requests += n > 0 ? 1 : 0;
  p->compared_tokens += n_tokens;
  p->hit_tokens += (int64_t)n * p->page;
  *n_match = n;
  return PKV_OK;
}

PKV_API int pkv_prefix_stats(const pkv_prefix* p, int64_t* hit_tokens, int64_t* compared_tokens,
                             int64_t* requests, int64_t* hit_requests, int32_t* num_entries) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_EINVAL, "pkv_prefix_stats: index is NULL");
  if (hit_tokens) *hit_tokens = p->hit_tokens;
  if (compared_tokens) *compared_tokens = p->compared_tokens;
  if (requests) *requests = p->requests;
  if (hit_requests) *hit_requests = p->hit_requests;
  if (num_entries) *num_entries = (int32_t)p->entries.size();
  return PKV_OK;
}

PKV_API int pkv_prefix_clear(pkv_prefix* p, pkv_alloc* alloc) {
  pkv::clear_error();
  if (!p) return pkv::fail(PKV_EINVAL, "pkv_prefix_clear: index is NULL");
  std::vector<int32_t> held;
  for (const Entry& e : p->entries)
    if (e.holds_ref) held.push_back(e.block);
  if (!held.empty()) {
    if (!alloc) return pkv::fail(PKV_EINVAL, "pkv_prefix_clear: indexed blocks hold allocator references; pass the allocator");
    if (int st = pkv_alloc_decref(alloc, held.data(), (int32_t)held.size())) return st;
  }
  p->entries.clear();
  p->tokens.clear();
  p->head.clear();
  return PKV_OK;
}

}  // extern "C"
