// The C ABI: argument validation, launch geometry, error reporting.
// Every entry point validates on the host first and launches nothing on error.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "errors.h"
#include "launch.h"

namespace pkv {

std::string& last_error() {
  thread_local std::string msg;
  return msg;
}

namespace {

// a wave reads its share of a partition's table entries one per lane
constexpr int32_t kMaxPartition = 64 * 16 * kDecodeWaves;
constexpr int64_t kMaxWorkgroups = INT32_MAX;   // one launch grid dimension
// MI355X compute units: the automatic partition size aims at one decode
// workgroup (8 waves, a whole CU at the kernel's register use) per CU
constexpr int32_t kComputeUnits = 256;
// below this many tokens a partition is not split further
constexpr int32_t kMinPartition = 256;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool check_mode() {
  const char* e = getenv("PKV_CHECK");
  return e && e[0] && strcmp(e, "0") != 0;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int validate_cache(const pkv_cache* c, const char* fn, CacheView* view) {
  const std::string f(fn);
  if (!c) return fail(PKV_EINVAL, f + ": cache is NULL");
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32 && c->block_size != 64)
    return fail(PKV_EINVAL, f + ": block_size must be 8, 16, 32 or 64");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(PKV_EINVAL, f + ": head_dim must be 64 or 128");
  if (c->num_kv_heads <= 0) return fail(PKV_EINVAL, f + ": num_kv_heads must be positive");
  if (c->num_blocks <= 0 || c->num_blocks > INT32_MAX / c->block_size)
    return fail(PKV_EINVAL, f + ": num_blocks out of range");
  if (c->dtype != PKV_F32 && c->dtype != PKV_BF16 && c->dtype != PKV_FP8_E4M3)
    return fail(PKV_EDTYPE, f + ": unknown cache dtype");
  if (!c->k_cache || !c->v_cache) return fail(PKV_EINVAL, f + ": k_cache / v_cache is NULL");
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache))
    return fail(PKV_EINVAL, f + ": k_cache / v_cache must be 16-byte aligned");
  if (c->dtype == PKV_FP8_E4M3 && (!c->k_scale || !c->v_scale))
    return fail(PKV_EINVAL, f + ": an fp8 cache needs k_scale and v_scale");
  view->num_blocks = c->num_blocks;
  view->num_kv_heads = c->num_kv_heads;
  view->head_dim = c->head_dim;
  view->dtype = c->dtype;
  view->block_size = c->block_size;
  view->k = c->k_cache;
  view->v = c->v_cache;
  view->k_scale = c->k_scale;
  view->v_scale = c->v_scale;
  return PKV_OK;
}

template <typename T>
int copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t s) {
  dst.resize(n);
  if (n == 0) return PKV_OK;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost);
  return hip_status(e, "PKV_CHECK copy");
}

// PKV_CHECK: every table entry a sequence will read names a pool block.
int check_tables(const std::vector<int32_t>& bt, int max_blocks, int seq, int tokens,
                 int num_blocks, const char* fn, int bs = 16) {
  const int nb = (tokens + bs - 1) / bs;
  if (nb > max_blocks) return fail(PKV_EINVAL, std::string(fn) + ": PKV_CHECK: sequence longer than its table");
  for (int i = 0; i < nb; ++i) {
    const int32_t id = bt[(size_t)seq * max_blocks + i];
    if (id < 0 || id >= num_blocks)
      return fail(PKV_EINVAL, std::string(fn) + ": PKV_CHECK: sequence " + std::to_string(seq) +
                                  " block " + std::to_string(i) + " has id " + std::to_string(id));
  }
  return PKV_OK;
}

// Partition size for pkv_attn_decode when the caller passes 0. A workgroup
// owns (sequence, KV head, chunk of up to 8 query heads, partition); with
// units = batch · Hkv · chunks, split each sequence into ceil(256 / units)
// partitions (one round of workgroups over the CUs, no split when the units
// already fill the chip), never below 256 tokens and never above the
// largest partition one workgroup can take.
// Which decode kernel runs: PKV_DECODE_KERNEL=vector|matrix overrides the
// default (the matrix kernel takes bf16 and fp8 caches only).
int decode_kernel_for(int32_t dtype) {
  if (dtype == PKV_F32) return kDecodeVector;
  const char* e = getenv("PKV_DECODE_KERNEL");
  if (e && std::string(e) == "vector") return kDecodeVector;
  return kDecodeMatrix;
}

int32_t auto_partition(int32_t batch, int32_t hq, int32_t hkv, int32_t max_seq_len, int kernel) {
  const int32_t msl16 = (std::max(max_seq_len, 1) + 15) / 16 * 16;
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv != 0) return std::min(msl16, kMaxPartition);
  const int group = hq / hkv;
  const int hpw = decode_heads_per_wg(group, kernel);
  const int64_t units = (int64_t)batch * hkv * ((group + hpw - 1) / hpw);
  const int64_t parts = std::max<int64_t>(1, (kComputeUnits + units - 1) / units);
  int32_t pt = (int32_t)(((max_seq_len + parts - 1) / parts + 15) / 16 * 16);
  pt = std::max(pt, std::min(kMinPartition, msl16));
  return std::min(pt, kMaxPartition);
}

int32_t effective_partition(int32_t batch, int32_t hq, int32_t hkv, int32_t max_seq_len, int32_t pt, int kernel) {
  return pt == 0 ? auto_partition(batch, hq, hkv, max_seq_len, kernel) : pt;
}

size_t decode_ws_bytes(int32_t batch, int32_t hq, int32_t dh, int32_t max_seq_len, int32_t pt) {
  if (batch <= 0 || hq <= 0 || max_seq_len <= 0 || pt <= 0) return 0;
  const int64_t parts = (max_seq_len + pt - 1) / pt;
  if (parts <= 1) return 0;
  const size_t rows = (size_t)batch * hq;
  return rows * parts * (dh + 2) * sizeof(float);
}

int check_append_dtypes(const CacheView& c, int32_t in_dtype, const float* k_inv, const float* v_inv,
                        const char* fn) {
  const bool ok_dtype = (c.dtype == PKV_F32 && in_dtype == PKV_F32) ||
                        (c.dtype == PKV_BF16 && in_dtype == PKV_BF16) ||
                        (c.dtype == PKV_FP8_E4M3 && (in_dtype == PKV_BF16 || in_dtype == PKV_F32));
  if (!ok_dtype) return fail(PKV_EDTYPE, std::string(fn) + ": input dtype does not match the cache");
  if (c.dtype == PKV_FP8_E4M3 && (!k_inv || !v_inv))
    return fail(PKV_EINVAL, std::string(fn) + ": fp8 cache needs k_inv_scale and v_inv_scale");
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" {

PKV_API int32_t pkv_version(void) { return 300; }

PKV_API const char* pkv_last_error(void) { return last_error().c_str(); }

PKV_API int pkv_slot_mapping(const int32_t* block_table, int32_t table_len, int32_t block_size,
                             int32_t first_pos, int32_t n, int32_t* out_slots) {
  clear_error();
  if (block_size <= 0 || n < 0 || first_pos < 0 || table_len < 0 || (n > 0 && (!block_table || !out_slots)))
    return fail(PKV_EINVAL, "pkv_slot_mapping: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    const int64_t pos = (int64_t)first_pos + i;
    const int64_t lb = pos / block_size;
    if (lb >= table_len) return fail(PKV_EINVAL, "pkv_slot_mapping: position beyond the block table");
    const int32_t phys = block_table[lb];
    if (phys < 0) return fail(PKV_EINVAL, "pkv_slot_mapping: position falls on an unallocated table entry");
    const int64_t slot = (int64_t)phys * block_size + pos % block_size;
    if (slot > INT32_MAX) return fail(PKV_EINVAL, "pkv_slot_mapping: slot overflows int32");
    out_slots[i] = (int32_t)slot;
  }
  return PKV_OK;
}

PKV_API int pkv_slot_mapping_device(const int32_t* block_tables, int32_t max_blocks,
                                    int32_t block_size, int32_t num_seqs, const int32_t* cu_new,
                                    const int32_t* first_pos, int32_t n_tokens, int32_t* out_slots,
                                    pkv_stream stream) {
  clear_error();
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64)
    return fail(PKV_EINVAL, "pkv_slot_mapping_device: block_size must be 8, 16, 32 or 64");
  if (num_seqs < 0 || n_tokens < 0 || max_blocks < 0) return fail(PKV_EINVAL, "pkv_slot_mapping_device: negative size");
  if (num_seqs > 0 && n_tokens > 0 && (!block_tables || !cu_new || !first_pos || !out_slots))
    return fail(PKV_EINVAL, "pkv_slot_mapping_device: NULL pointer");
  return hip_status(launch_slot_mapping(block_tables, max_blocks, block_size, num_seqs, cu_new, first_pos,
                                        n_tokens, out_slots, static_cast<hipStream_t>(stream)),
                    "pkv_slot_mapping_device");
}

PKV_API int pkv_kv_append(const pkv_cache* cache, const void* k_new, const void* v_new,
                          int32_t in_dtype, int32_t n_tokens, const int32_t* slot_mapping,
                          const float* k_inv_scale, const float* v_inv_scale, pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_kv_append", &c)) return st;
  if (n_tokens < 0) return fail(PKV_EINVAL, "pkv_kv_append: n_tokens < 0");
  if (n_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PKV_EINVAL, "pkv_kv_append: NULL pointer");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(PKV_EINVAL, "pkv_kv_append: k_new / v_new must be 16-byte aligned");
  if (int st = check_append_dtypes(c, in_dtype, k_inv_scale, v_inv_scale, "pkv_kv_append")) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    std::vector<int32_t> slots;
    if (int st = copy_to_host(slots, slot_mapping, (size_t)n_tokens, s)) return st;
    for (int32_t v : slots)
      if (v < -1 || (int64_t)v >= (int64_t)c.num_blocks * c.block_size)
        return fail(PKV_EINVAL, "pkv_kv_append: PKV_CHECK: slot " + std::to_string(v) + " outside the pool");
  }
  return hip_status(launch_kv_append(c, k_new, v_new, in_dtype, n_tokens, slot_mapping, k_inv_scale,
                                     v_inv_scale, s),
                    "pkv_kv_append");
}

PKV_API int pkv_kv_append_paged(const pkv_cache* cache, const void* k_new, const void* v_new,
                                int32_t in_dtype, int32_t num_seqs, const int32_t* cu_new,
                                const int32_t* first_pos, int32_t max_new, const int32_t* block_tables,
                                int32_t max_blocks, const float* k_inv_scale, const float* v_inv_scale,
                                int32_t* out_slots, pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_kv_append_paged", &c)) return st;
  if (num_seqs < 0 || max_new < 0 || max_blocks < 0) return fail(PKV_EINVAL, "pkv_kv_append_paged: negative size");
  if (num_seqs == 0 || max_new == 0) return PKV_OK;
  if (!k_new || !v_new || !cu_new || !first_pos || !block_tables)
    return fail(PKV_EINVAL, "pkv_kv_append_paged: NULL pointer");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(PKV_EINVAL, "pkv_kv_append_paged: k_new / v_new must be 16-byte aligned");
  if (int st = check_append_dtypes(c, in_dtype, k_inv_scale, v_inv_scale, "pkv_kv_append_paged")) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (check_mode()) {
    std::vector<int32_t> cu;
    if (int st = copy_to_host(cu, cu_new, (size_t)num_seqs + 1, s)) return st;
    if (cu[0] != 0) return fail(PKV_EINVAL, "pkv_kv_append_paged: PKV_CHECK: cu_new[0] != 0");
    for (int i = 0; i < num_seqs; ++i)
      if (cu[i + 1] < cu[i] || cu[i + 1] - cu[i] > max_new)
        return fail(PKV_EINVAL, "pkv_kv_append_paged: PKV_CHECK: sequence " + std::to_string(i) +
                                    " has a bad new-token count");
  }
  return hip_status(launch_kv_append_paged(c, k_new, v_new, in_dtype, num_seqs, cu_new, first_pos, max_new,
                                           block_tables, max_blocks, k_inv_scale, v_inv_scale, out_slots, s),
                    "pkv_kv_append_paged");
}

PKV_API size_t pkv_attn_decode_workspace_bytes(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                               int32_t partition_tokens) {
  const int32_t pt = effective_partition(batch, num_q_heads, num_kv_heads, max_seq_len, partition_tokens,
                                         decode_kernel_for(cache_dtype));
  return decode_ws_bytes(batch, num_q_heads, head_dim, max_seq_len, pt);
}

PKV_API int32_t pkv_attn_decode_auto_partition(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_seq_len) {
  return auto_partition(batch, num_q_heads, num_kv_heads, max_seq_len, decode_kernel_for(cache_dtype));
}

}  // extern "C"

struct NewTokens {   // the fused append's inputs
  const void* k_new;
  const void* v_new;
  int32_t in_dtype;
  const float* k_inv;
  const float* v_inv;
};

// Checks a decode call's arguments and fills *p (kernel chosen by the
// caller); p->batch == 0 means nothing to launch.
static int decode_prepare(const char* fn, const CacheView& c, const NewTokens* app, const void* q, int32_t q_dtype,
                          int32_t batch, int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* seq_lens, int32_t max_seq_len, float scale, int32_t partition_tokens,
                          float* out, void* workspace, size_t workspace_bytes, int kernel, hipStream_t s,
                          DecodeParams* p, bool static_scratch = false) {
  p->cache = c;
  p->batch = 0;
  p->num_q_heads = num_q_heads;
  p->max_blocks = max_blocks;
  p->kernel = kernel;
  p->num_parts = 1;
  p->part_tokens = 16;
  if (batch < 0 || num_q_heads <= 0 || max_blocks <= 0 || max_seq_len < 0)
    return fail(PKV_EINVAL, std::string(fn) + ": bad size");
  if (num_q_heads % c.num_kv_heads != 0) return fail(PKV_EINVAL, std::string(fn) + ": num_q_heads must be a multiple of num_kv_heads");
  if (num_q_heads / c.num_kv_heads > 64) return fail(PKV_EINVAL, std::string(fn) + ": more than 64 query heads per KV head");
  if ((int64_t)max_seq_len > (int64_t)max_blocks * c.block_size)
    return fail(PKV_EINVAL, std::string(fn) + ": max_seq_len exceeds max_blocks * block_size");
  if (partition_tokens != 0 && (partition_tokens < 16 || partition_tokens > kMaxPartition || partition_tokens % 16))
    return fail(PKV_EINVAL, std::string(fn) + ": partition_tokens must be 0 or a multiple of 16 in [16, " + std::to_string(kMaxPartition) + "]");
  const bool ok_q = (c.dtype == PKV_F32 && q_dtype == PKV_F32) ||
                    (c.dtype != PKV_F32 && q_dtype == PKV_BF16);
  if (!ok_q) return fail(PKV_EDTYPE, std::string(fn) + ": q dtype must be F32 for an F32 cache, BF16 otherwise");
  if (batch == 0) return PKV_OK;
  if (!q || !block_tables || !seq_lens || !out) return fail(PKV_EINVAL, std::string(fn) + ": NULL pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_EINVAL, std::string(fn) + ": q and out must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, std::string(fn) + ": scale is not finite");
  if (app) {
    if (int st = check_append_dtypes(c, app->in_dtype, app->k_inv, app->v_inv, fn)) return st;
    if (!app->k_new || !app->v_new) return fail(PKV_EINVAL, std::string(fn) + ": k_new / v_new is NULL");
    if (!aligned16(app->k_new) || !aligned16(app->v_new))
      return fail(PKV_EINVAL, std::string(fn) + ": k_new / v_new must be 16-byte aligned");
  }
  if (c.block_size != 16 && kernel != kDecodeMatrix)
    return fail(PKV_EINVAL, std::string(fn) + ": block sizes other than 16 need the matrix-core decode (bf16 or fp8 cache)");
  const int32_t pt = effective_partition(batch, num_q_heads, c.num_kv_heads, max_seq_len, partition_tokens, kernel);
  const int32_t parts = max_seq_len <= 0 ? 1 : (max_seq_len + pt - 1) / pt;
  {   // the split kernel's workgroups and the reduce kernel's rows must fit a launch grid
    const int group = num_q_heads / c.num_kv_heads;
    const int hpw = decode_heads_per_wg(group, kernel);
    const int64_t wgs = (int64_t)batch * c.num_kv_heads * ((group + hpw - 1) / hpw) * parts;
    if (wgs > kMaxWorkgroups || (int64_t)batch * num_q_heads > kMaxWorkgroups)
      return fail(PKV_EINVAL, std::string(fn) + ": batch x heads x partitions needs more than 2^31 - 1 workgroups");
  }
  const size_t need = decode_ws_bytes(batch, num_q_heads, c.head_dim, max_seq_len, pt);
  if (static_scratch && need > 0) {   // the library's static array instead of a caller's workspace
    if (need > kDecodeStaticScratchBytes)
      return fail(PKV_EWORKSPACE, std::string(fn) + ": the split-KV partials need " + std::to_string(need) +
                                      " bytes, more than the library's static scratch of " +
                                      std::to_string(kDecodeStaticScratchBytes) +
                                      " bytes; pass larger partitions or use pkv_attn_decode with a workspace");
    if (hipError_t e = decode_static_scratch(&workspace)) return hip_status(e, fn);
    workspace_bytes = kDecodeStaticScratchBytes;
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_EWORKSPACE, std::string(fn) + ": workspace needs " + std::to_string(need) + " bytes");
  if (need > 0 && !aligned16(workspace)) return fail(PKV_EINVAL, std::string(fn) + ": workspace must be 16-byte aligned");
  if (check_mode() && !static_scratch) {   // the no-allocation call skips the checking copies
    std::vector<int32_t> lens, bt;
    if (int st = copy_to_host(lens, seq_lens, (size_t)batch, s)) return st;
    if (int st = copy_to_host(bt, block_tables, (size_t)batch * max_blocks, s)) return st;
    for (int b = 0; b < batch; ++b) {
      if (lens[b] < 0 || lens[b] > max_seq_len)
        return fail(PKV_EINVAL, std::string(fn) + ": PKV_CHECK: seq_lens[" + std::to_string(b) + "] = " +
                                    std::to_string(lens[b]) + " outside [0, max_seq_len]");
      if (int st = check_tables(bt, max_blocks, b, lens[b], c.num_blocks, fn, c.block_size)) return st;
    }
  }
  p->q = q;
  p->batch = batch;
  p->max_seq_len = max_seq_len;
  p->part_tokens = pt;
  p->num_parts = parts;
  p->block_tables = block_tables;
  p->seq_lens = seq_lens;
  p->scale = scale;
  p->out = out;
  float* ws = static_cast<float*>(workspace);
  const size_t rows = (size_t)batch * num_q_heads;
  p->ws_u = need ? ws : nullptr;
  p->ws_ml = need ? ws + rows * parts * c.head_dim : nullptr;
  if (app && kernel == kDecodeMatrix) {   // the split kernel writes and reads the new tokens itself
    p->k_new = app->k_new;
    p->v_new = app->v_new;
    p->new_dtype = app->in_dtype;
    p->k_inv = app->k_inv;
    p->v_inv = app->v_inv;
  }
  return PKV_OK;
}

static int decode_impl(const char* fn, const pkv_cache* cache, const NewTokens* app, const void* q, int32_t q_dtype,
                       int32_t batch, int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* seq_lens, int32_t max_seq_len, float scale, int32_t partition_tokens,
                       float* out, void* workspace, size_t workspace_bytes, pkv_stream stream,
                       bool static_scratch = false) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, fn, &c)) return st;
  const int kernel = decode_kernel_for(c.dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  DecodeParams p;
  if (int st = decode_prepare(fn, c, app, q, q_dtype, batch, num_q_heads, block_tables, max_blocks, seq_lens,
                              max_seq_len, scale, partition_tokens, out, workspace, workspace_bytes, kernel, s, &p,
                              static_scratch))
    return st;
  if (p.batch == 0) return PKV_OK;
  if (app && kernel != kDecodeMatrix) {   // the vector form: an append launch first
    if (hipError_t e = launch_kv_append_last(c, app->k_new, app->v_new, app->in_dtype, batch, block_tables,
                                             max_blocks, seq_lens, max_seq_len, app->k_inv, app->v_inv, s))
      return hip_status(e, fn);
  }
  return hip_status(launch_decode(p, s), fn);
}

// The prefill kernel: the tile kernel (64 query rows of a KV group per
// workgroup, one workgroup per compute unit), or the matrix-core decode kernel
// with (head, query) columns (16 rows per workgroup, the keys split across
// its waves; tables of at most kPrefillColsMaxKeys tokens). The tile kernel
// is faster once the chunks give half the compute units their 64 rows
// (measured at Hq=32, Hkv=8 on 2048 cached tokens: C=256, 8192 rows, 37.9
// against 43.9 µs; C=128, 22.9 against 34.8 µs for the columns); below that
// the column form is used. Once the rows give every compute unit 128 of them,
// the tile kernel takes 128 rows per workgroup (two key streams of four
// waves: half the tile stream per product; C=1024 77.7 against 84.7 µs back
// to back, C=2048 160.8 against 178.3, C=4096 388.7 against 427.7 per call;
// at C=512 it would leave half the units idle), and once they give every unit
// two workgroups of 256 rows, 256 (one stream of eight waves, head dim 128;
// C=4096 363.4 against 378.7 µs; at C=2048 one round of them is slower,
// 180.8 against 161.3). PKV_PREFILL_KERNEL=tiles (64 rows), tiles128,
// tiles256, tiles16 or columns, read at every call, overrides the choice
// where it applies.
constexpr int64_t kPrefillTileRows = 128 * 64;
constexpr int64_t kPrefillTile128Rows = (int64_t)128 * kComputeUnits;
constexpr int64_t kPrefillTile256Rows = (int64_t)2 * 256 * kComputeUnits;
// The prefill kernel a call runs: the decode kernel's (head, query) columns
// for small chunks, the key-stream tile kernel with 64 rows per workgroup,
// or with 128 for large ones; PKV_PREFILL_KERNEL (tiles, tiles128, tiles16,
// columns) overrides.
enum PrefillKernel { kPrefillColumns, kPrefillTiles16, kPrefillStream, kPrefillStream128, kPrefillStream256 };
static PrefillKernel prefill_kernel_for(const PrefillParams& p) {
  // the column form and the 16-row tile kernel address 16-row units inside
  // blocks of 16 tokens or more; 8-token blocks take the key-stream kernel
  const bool cols_ok =
      p.cache.block_size >= 16 && (int64_t)p.max_blocks * p.cache.block_size <= kPrefillColsMaxKeys;
  const char* env = getenv("PKV_PREFILL_KERNEL");
  bool cols = cols_ok && (int64_t)p.num_seqs * p.max_q_len * p.num_q_heads < kPrefillTileRows;
  if (env && (strcmp(env, "tiles") == 0 || strcmp(env, "tiles16") == 0 || strcmp(env, "tiles128") == 0 ||
              strcmp(env, "tiles256") == 0))
    cols = false;
  if (env && strcmp(env, "columns") == 0) cols = cols_ok;
  if (cols) return kPrefillColumns;
  if (env && strcmp(env, "tiles16") == 0 && p.cache.block_size >= 16) return kPrefillTiles16;
  if (env && strcmp(env, "tiles128") == 0) return kPrefillStream128;
  if (env && strcmp(env, "tiles256") == 0) return kPrefillStream256;
  if (env && strcmp(env, "tiles") == 0) return kPrefillStream;
  const int64_t rows = (int64_t)p.num_seqs * p.max_q_len * p.num_q_heads;
  if (rows >= kPrefillTile256Rows && p.cache.head_dim == 128) return kPrefillStream256;
  return rows >= kPrefillTile128Rows ? kPrefillStream128 : kPrefillStream;
}

static hipError_t run_prefill(const PrefillParams& p, hipStream_t s) {
  switch (prefill_kernel_for(p)) {
    case kPrefillColumns: return launch_prefill_cols(p, s);
    case kPrefillTiles16: return launch_prefill(p, s);
    case kPrefillStream128: return launch_prefill_stream(p, 128, s);
    case kPrefillStream256: return launch_prefill_stream(p, 256, s);
    default: return launch_prefill_stream(p, 64, s);
  }
}

// Checks a prefill call's arguments and fills *p; p->num_seqs == 0 means
// nothing to launch.
static int prefill_prepare(const char* fn, const CacheView& c, const void* q, int32_t q_dtype, int32_t num_seqs,
                           int32_t num_q_heads, const int32_t* q_start, const int32_t* block_tables,
                           int32_t max_blocks, const int32_t* seq_lens, int32_t max_q_len, float scale, float* out,
                           hipStream_t s, PrefillParams* p) {
  p->num_seqs = 0;
  if (c.dtype != PKV_BF16 || q_dtype != PKV_BF16) return fail(PKV_EDTYPE, std::string(fn) + ": cache and q must be BF16");
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks <= 0 || max_q_len < 0)
    return fail(PKV_EINVAL, std::string(fn) + ": bad size");
  if (num_q_heads % c.num_kv_heads != 0)
    return fail(PKV_EINVAL, std::string(fn) + ": num_q_heads must be a multiple of num_kv_heads");
  const int group = num_q_heads / c.num_kv_heads;
  if (!(group == 1 || group == 2 || (group % 4 == 0 && group <= 64)))
    return fail(PKV_EINVAL, std::string(fn) + ": Hq/Hkv must be 1, 2 or a multiple of 4 up to 64");
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  // either kernel takes at least 16 (query head, query) rows per workgroup,
  // plus at most one partial query block per head group
  if ((int64_t)num_seqs * num_q_heads * (max_q_len / 16 + 1) > kMaxWorkgroups)
    return fail(PKV_EINVAL, std::string(fn) + ": sequences x heads x queries need more than 2^31 - 1 workgroups");
  if (!q || !q_start || !block_tables || !seq_lens || !out) return fail(PKV_EINVAL, std::string(fn) + ": NULL pointer");
  if (!aligned16(q) || !aligned16(out)) return fail(PKV_EINVAL, std::string(fn) + ": q and out must be 16-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PKV_EINVAL, std::string(fn) + ": scale must be positive and finite");
  if (check_mode()) {
    std::vector<int32_t> qs, lens, bt;
    if (int st = copy_to_host(qs, q_start, (size_t)num_seqs + 1, s)) return st;
    if (int st = copy_to_host(lens, seq_lens, (size_t)num_seqs, s)) return st;
    if (int st = copy_to_host(bt, block_tables, (size_t)num_seqs * max_blocks, s)) return st;
    if (qs[0] != 0) return fail(PKV_EINVAL, std::string(fn) + ": PKV_CHECK: q_start[0] != 0");
    for (int i = 0; i < num_seqs; ++i) {
      const int cq = qs[i + 1] - qs[i];
      if (cq < 0 || cq > max_q_len || lens[i] < cq || (int64_t)lens[i] > (int64_t)max_blocks * c.block_size)
        return fail(PKV_EINVAL, std::string(fn) + ": PKV_CHECK: bad q_start / seq_lens for sequence " + std::to_string(i));
      if (int st = check_tables(bt, max_blocks, i, lens[i], c.num_blocks, fn, c.block_size)) return st;
    }
  }
  p->cache = c;
  p->q = q;
  p->num_seqs = num_seqs;
  p->num_q_heads = num_q_heads;
  p->max_blocks = max_blocks;
  p->max_q_len = max_q_len;
  p->q_start = q_start;
  p->block_tables = block_tables;
  p->seq_lens = seq_lens;
  p->scale = scale;
  p->out = out;
  return PKV_OK;
}

extern "C" {

PKV_API int pkv_attn_decode(const pkv_cache* cache, const void* q, int32_t q_dtype, int32_t batch,
                            int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* seq_lens, int32_t max_seq_len, float scale,
                            int32_t partition_tokens, float* out, void* workspace,
                            size_t workspace_bytes, pkv_stream stream) {
  return decode_impl("pkv_attn_decode", cache, nullptr, q, q_dtype, batch, num_q_heads, block_tables, max_blocks,
                     seq_lens, max_seq_len, scale, partition_tokens, out, workspace, workspace_bytes, stream);
}

PKV_API int pkv_attn_decode_noalloc(const pkv_cache* cache, const void* q, int32_t q_dtype, int32_t batch,
                                    int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                                    const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                    int32_t partition_tokens, float* out, pkv_stream stream) {
  return decode_impl("pkv_attn_decode_noalloc", cache, nullptr, q, q_dtype, batch, num_q_heads, block_tables,
                     max_blocks, seq_lens, max_seq_len, scale, partition_tokens, out, nullptr, 0, stream, true);
}

PKV_API int pkv_attn_decode_append(const pkv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                                   const float* k_inv_scale, const float* v_inv_scale, const void* q,
                                   int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                   int32_t max_seq_len, float scale, int32_t partition_tokens, float* out,
                                   void* workspace, size_t workspace_bytes, pkv_stream stream) {
  const NewTokens app{k_new, v_new, in_dtype, k_inv_scale, v_inv_scale};
  return decode_impl("pkv_attn_decode_append", cache, &app, q, q_dtype, batch, num_q_heads, block_tables,
                     max_blocks, seq_lens, max_seq_len, scale, partition_tokens, out, workspace, workspace_bytes,
                     stream);
}

PKV_API int pkv_attn_prefill_chunk(const pkv_cache* cache, const void* q, int32_t q_dtype,
                                   int32_t num_seqs, int32_t num_q_heads, const int32_t* q_start,
                                   const int32_t* block_tables, int32_t max_blocks,
                                   const int32_t* seq_lens, int32_t max_q_len, float scale,
                                   float* out, pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_attn_prefill_chunk", &c)) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  PrefillParams p;
  if (int st = prefill_prepare("pkv_attn_prefill_chunk", c, q, q_dtype, num_seqs, num_q_heads, q_start, block_tables,
                               max_blocks, seq_lens, max_q_len, scale, out, s, &p))
    return st;
  if (p.num_seqs == 0) return PKV_OK;
  return hip_status(run_prefill(p, s), "pkv_attn_prefill_chunk");
}

PKV_API int pkv_attn_mixed_step(const pkv_cache* cache, int32_t num_q_heads, float scale,
                                const pkv_chunk_batch* chunks, const pkv_decode_batch* decodes,
                                pkv_stream stream) {
  const char* fn = "pkv_attn_mixed_step";
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, fn, &c)) return st;
  if (!chunks || !decodes) return fail(PKV_EINVAL, std::string(fn) + ": chunks / decodes is NULL");
  if (c.dtype != PKV_BF16) return fail(PKV_EDTYPE, std::string(fn) + ": the cache must be BF16");
  hipStream_t s = static_cast<hipStream_t>(stream);
  PrefillParams pp;
  if (int st = prefill_prepare(fn, c, chunks->q, PKV_BF16, chunks->num_seqs, num_q_heads, chunks->q_start,
                               chunks->block_tables, chunks->max_blocks, chunks->seq_lens, chunks->max_q_len, scale,
                               chunks->out, s, &pp))
    return st;
  if (pp.num_seqs > 0) {
    if (!chunks->k_new || !chunks->v_new) return fail(PKV_EINVAL, std::string(fn) + ": chunk k_new / v_new is NULL");
    if (!aligned16(chunks->k_new) || !aligned16(chunks->v_new))
      return fail(PKV_EINVAL, std::string(fn) + ": chunk k_new / v_new must be 16-byte aligned");
  }
  const NewTokens app{decodes->k_new, decodes->v_new, PKV_BF16, nullptr, nullptr};
  DecodeParams dp{};
  if (int st = decode_prepare(fn, c, &app, decodes->q, PKV_BF16, decodes->batch, num_q_heads, decodes->block_tables,
                              decodes->max_blocks, decodes->seq_lens, decodes->max_seq_len, scale,
                              decodes->partition_tokens, decodes->out, decodes->workspace, decodes->workspace_bytes,
                              kDecodeMatrix, s, &dp))
    return st;
  if (pp.num_seqs > 0) {   // the chunks' tokens: extra workgroups of the decode launch
    const int group = num_q_heads / c.num_kv_heads;
    const int hpw = decode_heads_per_wg(group, kDecodeMatrix);
    const int64_t dec_wgs = (int64_t)dp.batch * c.num_kv_heads * ((group + hpw - 1) / hpw) * dp.num_parts;
    const int64_t x_wgs = (int64_t)chunks->num_seqs * ((chunks->max_q_len + 15) / 16) + 8;
    if (dec_wgs + x_wgs > kMaxWorkgroups)
      return fail(PKV_EINVAL, std::string(fn) + ": the decode launch with its appending workgroups exceeds 2^31 - 1");
    dp.x_k = chunks->k_new;
    dp.x_v = chunks->v_new;
    dp.x_cu = chunks->q_start;
    dp.x_lens = chunks->seq_lens;
    dp.x_tables = chunks->block_tables;
    dp.x_max_blocks = chunks->max_blocks;
    dp.x_seqs = chunks->num_seqs;
    dp.x_max_q = chunks->max_q_len;
    dp.new_dtype = PKV_BF16;
    // One launch, paired (the default where it applies): four-wave
    // workgroups, a prefill tile and a decode workgroup on every CU, the
    // prefill waiting for the appends only where it reaches the chunk's own
    // keys (the shared-prefix step, a 512-token chunk on 2048 cached tokens
    // and 64 decodes: 80.0-80.8 us against 88.3-88.4 for two launches).
    // It needs the key-stream prefill's 64-row form on blocks of 16 tokens or
    // more and decode partitions of at most 4096 tokens. PKV_MIXED=two: two
    // launches (the decode launch with the appends, then the prefill),
    // bit-identical to the separate calls; PKV_MIXED=one: one launch of
    // eight-wave workgroups (the prefill after the decodes).
    // The paired launch pays only beside enough decode work (its prefill
    // tiles run at one wave per SIMD): by default it needs at least 2^20
    // (sequence, KV head, position) rows in the decodes' tables, as 64
    // decodes of up to 2048 tokens at Hkv=8 give. Measured on the shared-
    // prefix step (decode contexts up to 2048) against two launches: 32
    // decodes +3% (C=512) and +8% (C=128), one decode +20%; 64 decodes -9.5%
    // and -11%. PKV_MIXED=pair forces it.
    const char* menv = getenv("PKV_MIXED");
    const bool two = menv && strcmp(menv, "two") == 0;
    const bool one = menv && strcmp(menv, "one") == 0;
    const bool force_pair = menv && strcmp(menv, "pair") == 0;
    const bool enough_decodes = (int64_t)dp.batch * dp.max_seq_len * c.num_kv_heads >= ((int64_t)1 << 20);
    const bool pair = !two && !one && dp.part_tokens <= kMixedPairMaxPartition && (force_pair || enough_decodes);
    const PrefillKernel pk = prefill_kernel_for(pp);
    if ((one || pair) && pk == kPrefillStream && c.block_size >= 16)
      return hip_status(launch_mixed_one(dp, pp, pair, s), fn);
    // Small chunks, where the prefill alone takes the column form. Fewer than
    // 128 query blocks: appends, decodes and the query blocks in one launch of
    // the decode body (they fit in the decodes' ragged tail). More: the
    // paired launch with the key-stream tiles, whose idle CUs run the decodes
    // (unless PKV_PREFILL_KERNEL names a kernel). Measured on the
    // shared-prefix step with a C-token chunk (Hq=32, Hkv=8): C=32 53 us in
    // the first form against 56.5 paired and 64.4 in two launches; C=64 60 /
    // 59 / 66; C=128 63 paired against 68.7; C=192 65.4 against 86.8.
    if (!two && pk == kPrefillColumns) {
      const size_t qblocks = prefill_cols_workgroups(pp);
      if (qblocks > 0 && qblocks < 128) return hip_status(launch_mixed_cols(dp, pp, s), fn);
      if (pair && !getenv("PKV_PREFILL_KERNEL")) return hip_status(launch_mixed_one(dp, pp, true, s), fn);
    }
  }
  if (hipError_t e = launch_decode(dp, s)) return hip_status(e, fn);
  if (pp.num_seqs == 0) return PKV_OK;
  return hip_status(run_prefill(pp, s), fn);
}

PKV_API int pkv_copy_blocks(const pkv_cache* cache, const int32_t* src, const int32_t* dst, int32_t n,
                            pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_copy_blocks", &c)) return st;
  if (n < 0) return fail(PKV_EINVAL, "pkv_copy_blocks: n < 0");
  if (n == 0) return PKV_OK;
  if (!src || !dst) return fail(PKV_EINVAL, "pkv_copy_blocks: NULL pointer");
  return hip_status(launch_copy_blocks(c, src, dst, n, static_cast<hipStream_t>(stream)), "pkv_copy_blocks");
}

// Host buffer checks for the swap calls: large enough, 16-byte aligned and
// pinned (device-addressable) host memory, so the kernel never touches
// pageable memory.
static int check_swap_host(const CacheView& c, const void* host, size_t host_bytes, int32_t n, const char* what) {
  const size_t block_bytes = (size_t)c.num_kv_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  if (!host) return fail(PKV_EINVAL, std::string(what) + ": host is NULL");
  if (!aligned16(host)) return fail(PKV_EINVAL, std::string(what) + ": host must be 16-byte aligned");
  if (host_bytes < (size_t)n * 2 * block_bytes)
    return fail(PKV_EINVAL, std::string(what) + ": host buffer needs " + std::to_string((size_t)n * 2 * block_bytes) +
                                " bytes");
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, host) != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(PKV_EINVAL, std::string(what) + ": host must be pinned host memory (hipHostMalloc)");
  }
  return PKV_OK;
}

PKV_API int pkv_swap_out(const pkv_cache* cache, const int32_t* ids, int32_t n, void* host, size_t host_bytes,
                         pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_swap_out", &c)) return st;
  if (n < 0) return fail(PKV_EINVAL, "pkv_swap_out: n < 0");
  if (n == 0) return PKV_OK;
  if (!ids) return fail(PKV_EINVAL, "pkv_swap_out: ids is NULL");
  if (int st = check_swap_host(c, host, host_bytes, n, "pkv_swap_out")) return st;
  return hip_status(launch_swap_out(c, ids, n, host, static_cast<hipStream_t>(stream)), "pkv_swap_out");
}

PKV_API int pkv_swap_in(const pkv_cache* cache, const void* host, size_t host_bytes, const int32_t* ids, int32_t n,
                        pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_swap_in", &c)) return st;
  if (n < 0) return fail(PKV_EINVAL, "pkv_swap_in: n < 0");
  if (n == 0) return PKV_OK;
  if (!ids) return fail(PKV_EINVAL, "pkv_swap_in: ids is NULL");
  if (int st = check_swap_host(c, host, host_bytes, n, "pkv_swap_in")) return st;
  return hip_status(launch_swap_in(c, ids, n, host, static_cast<hipStream_t>(stream)),
                    "pkv_swap_in");
}

PKV_API int pkv_debug_gather(const pkv_cache* cache, const int32_t* block_table, int32_t seq_len,
                             void* k_out, void* v_out, pkv_stream stream) {
  clear_error();
  CacheView c;
  if (int st = validate_cache(cache, "pkv_debug_gather", &c)) return st;
  if (seq_len < 0) return fail(PKV_EINVAL, "pkv_debug_gather: seq_len < 0");
  if (seq_len == 0) return PKV_OK;
  if (!block_table || !k_out || !v_out) return fail(PKV_EINVAL, "pkv_debug_gather: NULL pointer");
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 3u)
    return fail(PKV_EINVAL, "pkv_debug_gather: outputs must be 4-byte aligned");
  return hip_status(launch_debug_gather(c, block_table, seq_len, k_out, v_out, static_cast<hipStream_t>(stream)),
                    "pkv_debug_gather");
}

PKV_API int pkv_debug_mfma_rate(const void* operands, int32_t iterations, int32_t num_workgroups, float* sink,
                                pkv_stream stream) {
  clear_error();
  const char* fn = "pkv_debug_mfma_rate";
  if (iterations < 0 || num_workgroups <= 0 || num_workgroups > kMaxWorkgroups)
    return fail(PKV_EINVAL, std::string(fn) + ": bad size");
  if (!operands || !sink) return fail(PKV_EINVAL, std::string(fn) + ": NULL pointer");
  if (!aligned16(operands)) return fail(PKV_EINVAL, std::string(fn) + ": operands must be 16-byte aligned");
  return hip_status(launch_mfma_rate(operands, iterations, num_workgroups, sink, static_cast<hipStream_t>(stream)),
                    fn);
}

PKV_API int pkv_debug_prefill_mix(const void* operands, const void* tiles, int64_t tiles_bytes, int32_t mode,
                                  int32_t iterations, int32_t num_workgroups, float* sink, pkv_stream stream) {
  clear_error();
  const char* fn = "pkv_debug_prefill_mix";
  if (iterations < 0 || num_workgroups <= 0 || num_workgroups > kMaxWorkgroups || mode < 0 || mode > 2)
    return fail(PKV_EINVAL, std::string(fn) + ": bad size or mode");
  if (tiles_bytes < kPrefillMixTileBytes) return fail(PKV_EINVAL, std::string(fn) + ": tiles must hold 1 MiB");
  if (!operands || !tiles || !sink) return fail(PKV_EINVAL, std::string(fn) + ": NULL pointer");
  if (!aligned16(operands) || !aligned16(tiles))
    return fail(PKV_EINVAL, std::string(fn) + ": operands and tiles must be 16-byte aligned");
  return hip_status(launch_prefill_mix(operands, tiles, mode, iterations, num_workgroups, sink,
                                       static_cast<hipStream_t>(stream)), fn);
}

PKV_API int pkv_debug_stream_read(const void* buf, int64_t buf_tiles, const int32_t* tile_ids, int32_t n_tiles,
                                  int32_t num_workgroups, uint32_t* sink, pkv_stream stream) {
  clear_error();
  const char* fn = "pkv_debug_stream_read";
  if (buf_tiles < 0 || n_tiles < 0 || num_workgroups <= 0 || num_workgroups > kMaxWorkgroups)
    return fail(PKV_EINVAL, std::string(fn) + ": bad size");
  if (n_tiles == 0) return PKV_OK;
  if (!buf || !tile_ids || !sink) return fail(PKV_EINVAL, std::string(fn) + ": NULL pointer");
  if (!aligned16(buf)) return fail(PKV_EINVAL, std::string(fn) + ": buf must be 16-byte aligned");
  return hip_status(launch_stream_read(buf, buf_tiles, tile_ids, n_tiles, num_workgroups, sink,
                                       static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
