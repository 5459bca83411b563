// Internal launcher interface between the C ABI (pkv_api.cpp) and the kernel
// translation units. Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

enum Dtype : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

inline int dtype_bytes(int dt) { return dt == kF32 ? 4 : dt == kBF16 ? 2 : 1; }

struct CacheView {
  int num_blocks, num_kv_heads, head_dim, dtype;
  int block_size;   // tokens per block: 8, 16, 32 or 64
  void* k;
  void* v;
  const float* k_scale;
  const float* v_scale;
};

hipError_t launch_slot_mapping(const int32_t* block_tables, int max_blocks, int block_size, int num_seqs,
                               const int32_t* cu_new, const int32_t* first_pos, int n_tokens,
                               int32_t* out_slots, hipStream_t s);

hipError_t launch_kv_append(const CacheView& c, const void* k_new, const void* v_new, int in_dtype,
                            int n_tokens, const int32_t* slots, const float* k_inv,
                            const float* v_inv, hipStream_t s);

hipError_t launch_kv_append_paged(const CacheView& c, const void* k_new, const void* v_new, int in_dtype,
                                  int num_seqs, const int32_t* cu_new, const int32_t* first_pos, int max_new,
                                  const int32_t* block_tables, int max_blocks, const float* k_inv,
                                  const float* v_inv, int32_t* out_slots, hipStream_t s);

hipError_t launch_copy_blocks(const CacheView& c, const int32_t* src, const int32_t* dst, int n,
                              hipStream_t s);

// Swap whole blocks between the pool and pinned host memory.
hipError_t launch_swap_out(const CacheView& c, const int32_t* ids, int n, void* host, hipStream_t s);
hipError_t launch_swap_in(const CacheView& c, const int32_t* ids, int n, const void* host, hipStream_t s);
hipError_t launch_debug_gather(const CacheView& c, const int32_t* table, int seq_len, void* k_out,
                               void* v_out, hipStream_t s);

// One new token per sequence appended at position seq_lens[s] − 1.
hipError_t launch_kv_append_last(const CacheView& c, const void* k_new, const void* v_new, int in_dtype, int batch,
                                 const int32_t* block_tables, int max_blocks, const int32_t* seq_lens,
                                 int max_seq_len, const float* k_inv, const float* v_inv, hipStream_t s);

struct DecodeParams {
  CacheView cache;
  const void* q;
  int batch, num_q_heads, max_blocks, max_seq_len, part_tokens, num_parts;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float scale;
  float* out;
  float* ws_u;         // [batch, Hq, num_parts, head_dim] (first in the workspace)
  float* ws_ml;        // [batch, Hq, num_parts, 2] (m, l) in log2 units
  int kernel;          // kDecodeVector or kDecodeMatrix
  // With k_new set (matrix kernel only), each sequence's new token k_new[b],
  // v_new[b] ([Hkv, head_dim] of new_dtype) is written to position
  // seq_lens[b] − 1 by the split kernel itself and attended to from k_new.
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int new_dtype = 0;
  const float* k_inv = nullptr;
  const float* v_inv = nullptr;
  // A mixed step's prefill-chunk tokens, appended by extra workgroups of the
  // same launch (matrix kernel, bf16 cache): sequence s's rows x_cu[s] …
  // x_cu[s+1]−1 of x_k / x_v go to its last x_cu[s+1] − x_cu[s] positions
  // (before x_lens[s]) through row s of x_tables; x_max_q bounds the rows
  // per sequence.
  const void* x_k = nullptr;
  const void* x_v = nullptr;
  const int32_t* x_cu = nullptr;
  const int32_t* x_lens = nullptr;
  const int32_t* x_tables = nullptr;
  int x_max_blocks = 0, x_seqs = 0, x_max_q = 0;
};

// Waves of one split-KV decode workgroup. A wave reads its share of the
// partition's table entries one per lane, so a partition holds at most
// 64 * kDecodeWaves blocks.
constexpr int kDecodeWaves = 8;

// The two decode kernels: products on the vector ALUs (any cache dtype), or
// on the matrix cores (bf16 and fp8 caches).
constexpr int kDecodeVector = 0;
constexpr int kDecodeMatrix = 1;

// Heads of one KV group handled by one decode workgroup of the given kernel.
int decode_heads_per_wg(int group, int kernel);
// Matrix-core rate probe (mfma_probe.hip): operands holds kMfmaProbeOperands
// bf16 values; sink num_wgs * 512 floats.
constexpr int kMfmaProbeOperands = 8 * (64 + 19);
hipError_t launch_mfma_rate(const void* operands, int iterations, int num_wgs, float* sink, hipStream_t s);
// The prefill's steady-iteration mix (mfma_probe.hip): tiles holds at least
// 1 MiB; mode 0, 1 or 2.
constexpr int kPrefillMixTileBytes = 1 << 20;
hipError_t launch_prefill_mix(const void* operands, const void* tiles, int mode, int iterations, int num_wgs,
                              float* sink, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t buf_tiles, const int32_t* ids, int n_tiles, int num_wgs,
                              uint32_t* sink, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);

// The library's own split-KV scratch for pkv_attn_decode_noalloc: a static
// device array of kDecodeStaticScratchBytes per GPU. *ptr receives its device
// address on the current device (looked up on the first call per device).
constexpr size_t kDecodeStaticScratchBytes = size_t(8) << 20;
hipError_t decode_static_scratch(void** ptr);

struct PrefillParams {
  CacheView cache;
  const void* q;
  int num_seqs, num_q_heads, max_blocks, max_q_len;
  const int32_t* q_start;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float scale;
  float* out;
};

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s);
// The mixed step in one launch: the chunks' appends, the decodes (each
// appending its token) and the chunks' prefill (key-stream form) in one grid;
// bf16 cache, matrix-core decode; the split-KV reduce follows when the decodes
// are split (see decode.hip). pair: four-wave workgroups, two per CU, the
// prefill tiles dispatched before the decodes so that each CU runs one of
// each (decode partitions of at most 4096 tokens).
hipError_t launch_mixed_one(const DecodeParams& dp, const PrefillParams& pp, bool pair, hipStream_t s);
// The mixed step in one launch when the prefill takes the column form (small
// chunks): appends, decodes, then the chunks' query blocks on the decode
// body; bit-identical to the separate calls.
hipError_t launch_mixed_cols(const DecodeParams& dp, const PrefillParams& pp, hipStream_t s);
// the column form's workgroups (query blocks) for a prefill call; 0 when the
// call does not fit the form
size_t prefill_cols_workgroups(const PrefillParams& p);
// the paired form's four-wave decode workgroups cover partitions of at most
// this many tokens (64 16-row units per wave; launch_mixed_one refuses more)
constexpr int kMixedPairMaxPartition = 64 * 16 * 4;
// The key-stream tile kernel: rows = 64 query rows per workgroup in four key
// streams of two 32-row waves, or 128 rows in two streams of four (see
// prefill_stream.h).
hipError_t launch_prefill_stream(const PrefillParams& p, int rows, hipStream_t s);

// The same chunked prefill on the matrix-core decode kernel: each workgroup
// takes 16 (query head, query) columns of one KV group — prefill_cols_heads
// heads × the rest in consecutive queries — over all the keys they see, split
// across its waves. Tables of at most kPrefillColsMaxKeys tokens.
constexpr int kPrefillColsMaxKeys = 8192;
int prefill_cols_heads(int group);
hipError_t launch_prefill_cols(const PrefillParams& p, hipStream_t s);

}  // namespace pkv
