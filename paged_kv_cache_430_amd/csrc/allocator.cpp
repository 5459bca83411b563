// Host block allocator with reference counts and copy-on-write of a shared
// partial tail.
//
// "07｜KV Cache、FlashAttention与PagedAttention的内部过程", Q028: blocks are
// taken on demand as a sequence grows and return to the pool when released;
// identical prefixes may share blocks with reference counts; writing into a
// shared, partly filled last block needs a private copy first (table row 6).
// "06 KV Cache…" 6.5: allocate on demand, map position to block and offset,
// grow, release or keep. "04. 注意力与 KV 缓存", engine section: a finished
// request must not free pages another one still uses.
#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "errors.h"

struct pkv_alloc {
  int32_t num_blocks;
  int32_t block_size;
  std::vector<int32_t> ref;
  std::vector<int32_t> free_stack;   // back() is handed out next
};

namespace {

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

extern "C" {

PKV_API int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                             pkv_alloc** out) {
  pkv::clear_error();
  if (!out) return pkv::fail(PKV_EINVAL, "pkv_alloc_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_create: num_blocks and block_size must be positive");
  pkv_alloc* a = new (std::nothrow) pkv_alloc;
  if (!a) return pkv::fail(PKV_EINVAL, "pkv_alloc_create: out of host memory");
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ref.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t id = free_order[i];
      if (id < 0 || id >= num_blocks || seen[id]) {
        delete a;
        return pkv::fail(PKV_EINVAL, "pkv_alloc_create: free_order is not a permutation of 0..num_blocks-1");
      }
      seen[id] = 1;
      a->free_stack[num_blocks - 1 - i] = id;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[num_blocks - 1 - i] = i;
  }
  *out = a;
  return PKV_OK;
}

PKV_API void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

PKV_API int pkv_alloc_allocate(pkv_alloc* a, int32_t n, int32_t* out_ids) {
  pkv::clear_error();
  if (!a || n < 0 || (n > 0 && !out_ids)) return pkv::fail(PKV_EINVAL, "pkv_alloc_allocate: bad argument");
  if ((size_t)n > a->free_stack.size())
    return pkv::fail(PKV_ENOBLOCKS, "pkv_alloc_allocate: not enough free blocks");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = a->free_stack.back();
    a->free_stack.pop_back();
    a->ref[id] = 1;
    out_ids[i] = id;
  }
  return PKV_OK;
}

PKV_API int pkv_alloc_incref(pkv_alloc* a, const int32_t* ids, int32_t n) {
  pkv::clear_error();
  if (!a || n < 0 || (n > 0 && !ids)) return pkv::fail(PKV_EINVAL, "pkv_alloc_incref: bad argument");
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= a->num_blocks) return pkv::fail(PKV_EINVAL, "pkv_alloc_incref: id outside the pool");
  for (int32_t i = 0; i < n; ++i)
    if (a->ref[ids[i]] <= 0) return pkv::fail(PKV_EREF, "pkv_alloc_incref: block is free");
  for (int32_t i = 0; i < n; ++i) ++a->ref[ids[i]];
  return PKV_OK;
}

PKV_API int pkv_alloc_decref(pkv_alloc* a, const int32_t* ids, int32_t n) {
  pkv::clear_error();
  if (!a || n < 0 || (n > 0 && !ids)) return pkv::fail(PKV_EINVAL, "pkv_alloc_decref: bad argument");
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= a->num_blocks) return pkv::fail(PKV_EINVAL, "pkv_alloc_decref: id outside the pool");
  std::unordered_map<int32_t, int32_t> need;
  for (int32_t i = 0; i < n; ++i) ++need[ids[i]];
  for (const auto& kv : need)
    if (a->ref[kv.first] < kv.second) return pkv::fail(PKV_EREF, "pkv_alloc_decref: reference count would drop below zero");
  for (int32_t i = 0; i < n; ++i) {
    if (--a->ref[ids[i]] == 0) a->free_stack.push_back(ids[i]);
  }
  return PKV_OK;
}

PKV_API int pkv_alloc_refcount(const pkv_alloc* a, int32_t id) {
  pkv::clear_error();
  if (!a || id < 0 || id >= a->num_blocks) return pkv::fail(PKV_EINVAL, "pkv_alloc_refcount: bad id");
  return a->ref[id];
}

PKV_API int32_t pkv_alloc_num_free(const pkv_alloc* a) {
  return a ? (int32_t)a->free_stack.size() : 0;
}

PKV_API int pkv_alloc_reserve_append(pkv_alloc* a, int32_t* table, int32_t max_blocks,
                                     int32_t seq_len, int32_t n_new, int32_t* cow_src,
                                     int32_t* cow_dst, int32_t* n_cow) {
  pkv::clear_error();
  if (!a || !table || max_blocks < 0 || seq_len < 0 || n_new < 0 || !n_cow)
    return pkv::fail(PKV_EINVAL, "pkv_alloc_reserve_append: bad argument");
  *n_cow = 0;
  const int32_t bs = a->block_size;
  const int32_t have = ceil_div(seq_len, bs);
  const int64_t need64 = ((int64_t)seq_len + n_new + bs - 1) / bs;
  if (need64 > max_blocks) return pkv::fail(PKV_EINVAL, "pkv_alloc_reserve_append: table too short");
  const int32_t need = (int32_t)need64;
  for (int32_t lb = 0; lb < have; ++lb)
    if (table[lb] < 0 || table[lb] >= a->num_blocks || a->ref[table[lb]] <= 0)
      return pkv::fail(PKV_EINVAL, "pkv_alloc_reserve_append: table holds an invalid or free block");
  const bool cow = n_new > 0 && seq_len % bs != 0 && a->ref[table[have - 1]] > 1;
  if (cow && (!cow_src || !cow_dst)) return pkv::fail(PKV_EINVAL, "pkv_alloc_reserve_append: cow arrays are NULL");
  const int32_t fresh = need - have;
  if ((size_t)(fresh + (cow ? 1 : 0)) > a->free_stack.size())
    return pkv::fail(PKV_ENOBLOCKS, "pkv_alloc_reserve_append: not enough free blocks");
  if (cow) {
    const int32_t src = table[have - 1];
    const int32_t dst = a->free_stack.back();
    a->free_stack.pop_back();
    a->ref[dst] = 1;
    --a->ref[src];                      // stays > 0: the block was shared
    table[have - 1] = dst;
    cow_src[0] = src;
    cow_dst[0] = dst;
    *n_cow = 1;
  }
  for (int32_t lb = have; lb < need; ++lb) {
    const int32_t id = a->free_stack.back();
    a->free_stack.pop_back();
    a->ref[id] = 1;
    table[lb] = id;
  }
  return PKV_OK;
}

}  // extern "C"
