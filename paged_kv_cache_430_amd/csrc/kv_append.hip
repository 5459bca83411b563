// Slot mapping, KV append (copy or e4m3 quantise), copy-on-write block copy
// and the test-only gather, for gfx950.
//
// Paging arithmetic follows "07｜KV Cache、FlashAttention与PagedAttention的内部过程",
// Q028 (block-size-4 table): position p → logical block p / bs, offset p % bs,
// physical block from the table; slot = physical * bs + offset. The append
// order (write the new token's K/V, then attend) follows Q025's "generate a
// new token" paragraph and "06 KV Cache…" section 6.1.
#include "append_common.h"
#include "device_common.h"
#include "launch.h"

namespace pkv {

// ---------------------------------------------------------------------------
// slot mapping: one workgroup per sequence, threads stride over its new tokens
// ---------------------------------------------------------------------------
__global__ void slot_mapping_kernel(const int32_t* __restrict__ block_tables, int max_blocks,
                                    const int32_t* __restrict__ cu_new,
                                    const int32_t* __restrict__ first_pos, int n_tokens, int bs,
                                    int32_t* __restrict__ out) {
  const int s = blockIdx.x;
  const int lo = cu_new[s];
  const int hi = min(cu_new[s + 1], n_tokens);
  const int p0 = first_pos[s];
  const int32_t* bt = block_tables + (size_t)s * max_blocks;
  for (int i = lo + (int)threadIdx.x; i < hi; i += blockDim.x) out[i] = slot_of(bt, max_blocks, p0 + (i - lo), bs);
}

hipError_t launch_slot_mapping(const int32_t* block_tables, int max_blocks, int block_size, int num_seqs,
                               const int32_t* cu_new, const int32_t* first_pos, int n_tokens,
                               int32_t* out_slots, hipStream_t s) {
  if (num_seqs == 0 || n_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_seqs), dim3(128), 0, s, block_tables,
                     max_blocks, cu_new, first_pos, n_tokens, block_size, out_slots);
  return hipGetLastError();
}

// One workgroup per token.
template <int IN, int OUT>
__global__ void kv_append_kernel(const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
                                 const int32_t* __restrict__ slots, uint8_t* __restrict__ kc,
                                 uint8_t* __restrict__ vc, int num_blocks, int hkv, int dh,
                                 const float* __restrict__ k_inv, const float* __restrict__ v_inv, int bs) {
  const int tok = blockIdx.x;
  append_token<IN, OUT>(k_new, v_new, tok, slots[tok], kc, vc, num_blocks, hkv, dh, k_inv, v_inv,
                        threadIdx.x, blockDim.x, bs);
}

// Slot mapping fused into the append: workgroup (s, j) takes sequence s's new
// tokens j·kAppendTokensPerWg … +kAppendTokensPerWg−1, each handled by a
// quarter of the workgroup; the slot comes from the table as in
// slot_mapping_kernel and is optionally written out.
constexpr int kAppendTokensPerWg = 4;
template <int IN, int OUT>
__global__ void kv_append_paged_kernel(const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
                                       const int32_t* __restrict__ block_tables, int max_blocks,
                                       const int32_t* __restrict__ cu_new,
                                       const int32_t* __restrict__ first_pos, uint8_t* __restrict__ kc,
                                       uint8_t* __restrict__ vc, int num_blocks, int hkv, int dh,
                                       const float* __restrict__ k_inv, const float* __restrict__ v_inv,
                                       int32_t* __restrict__ out_slots, int bs) {
  const int s = blockIdx.x;
  const int lo = cu_new[s], hi = cu_new[s + 1];
  const int part = threadIdx.x / (blockDim.x / kAppendTokensPerWg);
  const int nt = blockDim.x / kAppendTokensPerWg;
  const int i = lo + blockIdx.y * kAppendTokensPerWg + part;
  if (i >= hi) return;
  const int slot = slot_of(block_tables + (size_t)s * max_blocks, max_blocks, first_pos[s] + (i - lo), bs);
  if (out_slots && threadIdx.x % nt == 0) out_slots[i] = slot;
  append_token<IN, OUT>(k_new, v_new, i, slot, kc, vc, num_blocks, hkv, dh, k_inv, v_inv, threadIdx.x % nt, nt, bs);
}

hipError_t launch_kv_append(const CacheView& c, const void* k_new, const void* v_new, int in_dtype,
                            int n_tokens, const int32_t* slots, const float* k_inv,
                            const float* v_inv, hipStream_t s) {
  if (n_tokens == 0) return hipSuccess;
  const dim3 grid(n_tokens), block(128);
  auto kn = static_cast<const uint8_t*>(k_new);
  auto vn = static_cast<const uint8_t*>(v_new);
  auto kc = static_cast<uint8_t*>(c.k);
  auto vc = static_cast<uint8_t*>(c.v);
#define PKV_APPEND(IN, OUT)                                                                      \
  hipLaunchKernelGGL((kv_append_kernel<IN, OUT>), grid, block, 0, s, kn, vn, slots, kc, vc,      \
                     c.num_blocks, c.num_kv_heads, c.head_dim, k_inv, v_inv, c.block_size)
  if (c.dtype == kF32) PKV_APPEND(kF32, kF32);
  else if (c.dtype == kBF16) PKV_APPEND(kBF16, kBF16);
  else if (in_dtype == kBF16) PKV_APPEND(kBF16, kFP8);
  else PKV_APPEND(kF32, kFP8);
#undef PKV_APPEND
  return hipGetLastError();
}

// One new token per sequence at position T − 1 (T = seq_lens[s] clamped as
// the decode clamps it): workgroup s appends k_new[s], v_new[s].
template <int IN, int OUT>
__global__ void kv_append_last_kernel(const uint8_t* __restrict__ k_new, const uint8_t* __restrict__ v_new,
                                      const int32_t* __restrict__ block_tables, int max_blocks,
                                      const int32_t* __restrict__ seq_lens, int max_seq_len,
                                      uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, int num_blocks, int hkv,
                                      int dh, const float* __restrict__ k_inv, const float* __restrict__ v_inv,
                                      int bs) {
  const int s = blockIdx.x;
  const int T = min(max(seq_lens[s], 0), min(max_seq_len, max_blocks * bs));
  if (T <= 0) return;
  const int slot = slot_of(block_tables + (size_t)s * max_blocks, max_blocks, T - 1, bs);
  append_token<IN, OUT>(k_new, v_new, s, slot, kc, vc, num_blocks, hkv, dh, k_inv, v_inv, threadIdx.x, blockDim.x,
                        bs);
}

hipError_t launch_kv_append_last(const CacheView& c, const void* k_new, const void* v_new, int in_dtype, int batch,
                                 const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                                 int max_seq_len, const float* k_inv, const float* v_inv, hipStream_t s) {
  if (batch == 0) return hipSuccess;
  auto kn = static_cast<const uint8_t*>(k_new);
  auto vn = static_cast<const uint8_t*>(v_new);
  auto kc = static_cast<uint8_t*>(c.k);
  auto vc = static_cast<uint8_t*>(c.v);
#define PKV_APPEND(IN, OUT)                                                                                   \
  hipLaunchKernelGGL((kv_append_last_kernel<IN, OUT>), dim3(batch), dim3(128), 0, s, kn, vn, block_tables,    \
                     max_blocks, seq_lens, max_seq_len, kc, vc, c.num_blocks, c.num_kv_heads, c.head_dim, k_inv, \
                     v_inv, c.block_size)
  if (c.dtype == kF32) PKV_APPEND(kF32, kF32);
  else if (c.dtype == kBF16) PKV_APPEND(kBF16, kBF16);
  else if (in_dtype == kBF16) PKV_APPEND(kBF16, kFP8);
  else PKV_APPEND(kF32, kFP8);
#undef PKV_APPEND
  return hipGetLastError();
}

hipError_t launch_kv_append_paged(const CacheView& c, const void* k_new, const void* v_new, int in_dtype,
                                  int num_seqs, const int32_t* cu_new, const int32_t* first_pos, int max_new,
                                  const int32_t* block_tables, int max_blocks, const float* k_inv,
                                  const float* v_inv, int32_t* out_slots, hipStream_t s) {
  if (num_seqs == 0 || max_new == 0) return hipSuccess;
  const dim3 grid(num_seqs, (max_new + kAppendTokensPerWg - 1) / kAppendTokensPerWg), block(256);
  auto kn = static_cast<const uint8_t*>(k_new);
  auto vn = static_cast<const uint8_t*>(v_new);
  auto kc = static_cast<uint8_t*>(c.k);
  auto vc = static_cast<uint8_t*>(c.v);
#define PKV_APPEND(IN, OUT)                                                                             \
  hipLaunchKernelGGL((kv_append_paged_kernel<IN, OUT>), grid, block, 0, s, kn, vn, block_tables, max_blocks, \
                     cu_new, first_pos, kc, vc, c.num_blocks, c.num_kv_heads, c.head_dim, k_inv, v_inv,   \
                     out_slots, c.block_size)
  if (c.dtype == kF32) PKV_APPEND(kF32, kF32);
  else if (c.dtype == kBF16) PKV_APPEND(kBF16, kBF16);
  else if (in_dtype == kBF16) PKV_APPEND(kBF16, kFP8);
  else PKV_APPEND(kF32, kFP8);
#undef PKV_APPEND
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// copy-on-write: whole blocks, all heads, K and V; one workgroup per pair
// ---------------------------------------------------------------------------
__global__ void copy_blocks_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                   const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                                   int num_blocks, size_t block_bytes) {
  const int i = blockIdx.x;
  const int s = src[i], d = dst[i];
  if ((unsigned)s >= (unsigned)num_blocks || (unsigned)d >= (unsigned)num_blocks) return;
  const size_t n16 = block_bytes / 16;
  for (size_t c = threadIdx.x; c < 2 * n16; c += blockDim.x) {
    uint8_t* base = c < n16 ? kc : vc;
    const size_t cc = c < n16 ? c : c - n16;
    const uint4 x = reinterpret_cast<const uint4*>(base + (size_t)s * block_bytes)[cc];
    reinterpret_cast<uint4*>(base + (size_t)d * block_bytes)[cc] = x;
  }
}

hipError_t launch_copy_blocks(const CacheView& c, const int32_t* src, const int32_t* dst, int n,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t block_bytes = (size_t)c.num_kv_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(256), 0, s, static_cast<uint8_t*>(c.k),
                     static_cast<uint8_t*>(c.v), src, dst, c.num_blocks, block_bytes);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// swap-out / swap-in between the pool and pinned host memory: one workgroup
// per listed block; host slot i holds block ids[i] as its K bytes then its V
// bytes. The kernel itself moves the data across the host link (the host
// buffer is pinned and device-addressable), so scattered ids need no staging.
// ---------------------------------------------------------------------------
__global__ void swap_out_kernel(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                                const int32_t* __restrict__ ids, int num_blocks, size_t block_bytes,
                                uint8_t* __restrict__ host) {
  const int i = blockIdx.x;
  const int b = ids[i];
  if ((unsigned)b >= (unsigned)num_blocks) return;       // left untouched
  const size_t n16 = block_bytes / 16;
  uint4* dst = reinterpret_cast<uint4*>(host + (size_t)i * 2 * block_bytes);
  const uint4* ks = reinterpret_cast<const uint4*>(kc + (size_t)b * block_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(vc + (size_t)b * block_bytes);
  for (size_t c = threadIdx.x; c < n16; c += blockDim.x) {
    dst[c] = ks[c];
    dst[n16 + c] = vs[c];
  }
}

__global__ void swap_in_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                               const int32_t* __restrict__ ids, int num_blocks, size_t block_bytes,
                               const uint8_t* __restrict__ host) {
  const int i = blockIdx.x;
  const int b = ids[i];
  if ((unsigned)b >= (unsigned)num_blocks) return;       // skipped
  const size_t n16 = block_bytes / 16;
  const uint4* src = reinterpret_cast<const uint4*>(host + (size_t)i * 2 * block_bytes);
  uint4* kd = reinterpret_cast<uint4*>(kc + (size_t)b * block_bytes);
  uint4* vd = reinterpret_cast<uint4*>(vc + (size_t)b * block_bytes);
  for (size_t c = threadIdx.x; c < n16; c += blockDim.x) {
    kd[c] = src[c];
    vd[c] = src[n16 + c];
  }
}

hipError_t launch_swap_out(const CacheView& c, const int32_t* ids, int n, void* host, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t block_bytes = (size_t)c.num_kv_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  hipLaunchKernelGGL(swap_out_kernel, dim3(n), dim3(256), 0, s, static_cast<const uint8_t*>(c.k),
                     static_cast<const uint8_t*>(c.v), ids, c.num_blocks, block_bytes, static_cast<uint8_t*>(host));
  return hipGetLastError();
}

hipError_t launch_swap_in(const CacheView& c, const int32_t* ids, int n, const void* host, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t block_bytes = (size_t)c.num_kv_heads * c.block_size * c.head_dim * dtype_bytes(c.dtype);
  hipLaunchKernelGGL(swap_in_kernel, dim3(n), dim3(256), 0, s, static_cast<uint8_t*>(c.k), static_cast<uint8_t*>(c.v),
                     ids, c.num_blocks, block_bytes, static_cast<const uint8_t*>(host));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// test aid: paged → [Hkv, T, Dh] through the same slot arithmetic
// ---------------------------------------------------------------------------
__global__ void debug_gather_kernel(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                                    const int32_t* __restrict__ table, int seq_len, int num_blocks,
                                    int hkv, int row_bytes, uint8_t* __restrict__ k_out,
                                    uint8_t* __restrict__ v_out, int bs) {
  const int p = blockIdx.x;
  const int h = blockIdx.y;
  const int phys = table[p / bs];
  if ((unsigned)phys >= (unsigned)num_blocks) return;
  const size_t src = (((size_t)phys * hkv + h) * bs + p % bs) * row_bytes;
  const size_t dst = ((size_t)h * seq_len + p) * row_bytes;
  for (int b = threadIdx.x * 4; b < row_bytes; b += blockDim.x * 4) {
    *reinterpret_cast<uint32_t*>(k_out + dst + b) = *reinterpret_cast<const uint32_t*>(kc + src + b);
    *reinterpret_cast<uint32_t*>(v_out + dst + b) = *reinterpret_cast<const uint32_t*>(vc + src + b);
  }
}

hipError_t launch_debug_gather(const CacheView& c, const int32_t* table, int seq_len, void* k_out,
                               void* v_out, hipStream_t s) {
  if (seq_len == 0) return hipSuccess;
  const int row_bytes = c.head_dim * dtype_bytes(c.dtype);
  hipLaunchKernelGGL(debug_gather_kernel, dim3(seq_len, c.num_kv_heads), dim3(64), 0, s,
                     static_cast<const uint8_t*>(c.k), static_cast<const uint8_t*>(c.v), table,
                     seq_len, c.num_blocks, c.num_kv_heads, row_bytes,
                     static_cast<uint8_t*>(k_out), static_cast<uint8_t*>(v_out), c.block_size);
  return hipGetLastError();
}

}  // namespace pkv
