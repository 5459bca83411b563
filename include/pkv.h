/*
 * pkv.h — paged KV-cache attention for AMD MI355X (gfx950): the C ABI.
 *
 * What the library computes. New queries attend to keys and values that a
 * sequence has cached, stored in fixed-size blocks of a shared pool and found
 * through the sequence's block table, with an online (running max / running
 * sum) softmax. Sources, by page title and section:
 *   [P1] "04. 注意力与 KV 缓存" (niuwancheng.cn, inference series 04)
 *   [P2] "07｜KV Cache、FlashAttention与PagedAttention的内部过程"
 *        (ai-engineering-handbook.eonloom.com, chapter 07), Q025–Q028
 *   [P3] "06 KV Cache、Prefix Cache、PagedAttention 与 vLLM", sections 6.1–6.7
 *   [P4] "03. KV Cache：用显存换计算" (niuwancheng.cn, llm-inference 03)
 *
 * Conventions for every call:
 *   - Every call returns a pkv_status (0 = ok, negative = error); the reason
 *     of the last failure on the calling thread is in pkv_last_error().
 *     No C++ exception crosses this boundary.
 *   - Device pointers are caller-owned (allocated by the caller, e.g. by
 *     PyTorch). The library never allocates or frees device memory.
 *   - Kernels are launched asynchronously on the caller's stream (a
 *     hipStream_t passed as void*; NULL is the default stream). The caller
 *     owns synchronisation. A launch failure returns PKV_EHIP.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call launches nothing. Table ids and lengths that live in
 *     device memory are not read on the host unless the environment sets
 *     PKV_CHECK=1, in which case they are copied back (synchronously) and
 *     range-checked first. Without that check, kernels still never touch
 *     memory outside the pool: an out-of-range block id contributes nothing
 *     and an out-of-range slot is skipped.
 *   - Pool layout: K and V each [num_blocks, num_kv_heads, block_size,
 *     head_dim], row-major, in the cache dtype. The flat slot of a token is
 *     physical_block * block_size + offset ([P2] Q028 block-size-4 table).
 *   - GQA grouping: query head h reads KV head h / (Hq / Hkv) (contiguous
 *     groups; [P3] 6.3 says query heads share KV heads without fixing the
 *     order). MHA has Hq == Hkv, MQA has Hkv == 1.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_API __attribute__((visibility("default")))

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = -1,      /* bad shape, size, pointer or id; also an attention  */
                        /* call whose launch would need more than 2^31 - 1    */
                        /* workgroups                                          */
  PKV_ENOBLOCKS = -2,   /* allocator: not enough free blocks (state unchanged) */
  PKV_EDTYPE = -3,      /* unsupported dtype combination                       */
  PKV_EREF = -4,        /* allocator: reference count misuse                   */
  PKV_EWORKSPACE = -5,  /* workspace missing or too small                      */
  PKV_EHIP = -6         /* a HIP runtime call or kernel launch failed          */
} pkv_status;

typedef enum pkv_dtype {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  PKV_FP8_E4M3 = 2      /* OCP e4m3fn bytes with one fp32 scale per KV head    */
} pkv_dtype;

typedef void* pkv_stream;   /* a hipStream_t */

/* One layer's paged cache. Borrowed: the library keeps no pointer past a call.
 * Supported: block_size 8, 16, 32 or 64; head_dim 64 or 128; dtype F32, BF16 or
 * FP8_E4M3. Every call takes 8-, 16-, 32- and 64-token blocks except the F32
 * decode (its vector-ALU kernel, 16 only). [P2]
 * Q028 leaves the block size to the implementation and, in its follow-up on
 * smaller blocks, names the trade: a larger block wastes more tail slots
 * (blocks·bs − T) but needs fewer table entries and lookups.
 * k_scale/v_scale: device fp32 [num_kv_heads], the dequantisation scale of
 * each KV head (stored byte decoded, times scale, is the value attended to);
 * required for FP8_E4M3, ignored otherwise. */
typedef struct pkv_cache {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;            /* pkv_dtype of the stored values */
  void* k_cache;            /* device */
  void* v_cache;            /* device */
  const float* k_scale;     /* device [num_kv_heads] or NULL */
  const float* v_scale;     /* device [num_kv_heads] or NULL */
} pkv_cache;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
PKV_API int32_t pkv_version(void);

/* Reason for the last non-OK status returned on this thread ("" if none).
 * The string stays valid until the next pkv_* call on the same thread. */
PKV_API const char* pkv_last_error(void);

/* ---------------------------------------------------------------------------
 * Slot mapping — [P2] Q028, table "which physical slot logical position 5
 * maps to": a logical position p lives in logical block p / bs at offset
 * p % bs; the block table names the physical block; [P3] 6.5 gives the same
 * flow (position → logical block and offset → kernel reads through the table).
 * slot = block_table[p / bs] * bs + p % bs.
 * ------------------------------------------------------------------------- */

/* Host helper. block_table: host int32 [table_len]; writes n slots for the
 * positions first_pos … first_pos+n-1 into host out_slots[n].
 * PKV_EINVAL if a position falls beyond table_len blocks or on a negative
 * table entry, or if block_size <= 0 / n < 0 / first_pos < 0. */
PKV_API int pkv_slot_mapping(const int32_t* block_table, int32_t table_len, int32_t block_size,
                             int32_t first_pos, int32_t n, int32_t* out_slots);

/* Device variant for a batch. Sequence s appends new tokens
 * cu_new[s] … cu_new[s+1]-1 at logical positions first_pos[s], first_pos[s]+1, …
 *   block_tables: device int32 [num_seqs, max_blocks] (−1 = unused entry)
 *   cu_new:       device int32 [num_seqs + 1], nondecreasing, cu_new[0] = 0
 *   first_pos:    device int32 [num_seqs]
 *   out_slots:    device int32 [n_tokens] (n_tokens = cu_new[num_seqs])
 * A token whose logical block is beyond max_blocks or whose table entry is
 * negative gets slot −1 (skipped by pkv_kv_append). */
PKV_API int pkv_slot_mapping_device(const int32_t* block_tables, int32_t max_blocks,
                                    int32_t block_size, int32_t num_seqs, const int32_t* cu_new,
                                    const int32_t* first_pos, int32_t n_tokens,
                                    int32_t* out_slots, pkv_stream stream);

/* ---------------------------------------------------------------------------
 * KV append — [P2] Q025 core answer and "generate a new token" paragraph:
 * in every layer the new token's k and v are appended to that layer's cache
 * before its query attends; [P3] 6.1 (compute q/k/v → rotate → append k/v →
 * attend); [P4] lifecycle stage "fill" (prefill writes the prompt's K/V, each
 * decode step appends one token's).
 *
 * k_new, v_new: device [n_tokens, num_kv_heads, head_dim] in in_dtype.
 * slot_mapping: device int32 [n_tokens]; slot −1 (or any slot outside the
 *   pool) skips the token.
 * Stored value: F32→F32 and BF16→BF16 copy bit for bit; BF16 or F32 input
 *   into an FP8_E4M3 cache stores e4m3(fp32(x) · inv_scale[h]) with round to
 *   nearest even and saturation at ±448 (NaN stays NaN).
 * k_inv_scale, v_inv_scale: device fp32 [num_kv_heads], FP8 caches only
 *   (normally fp32(1 / scale) so that dequantisation inverts quantisation).
 * Two tokens with the same slot in one call race (the pages never write one
 * slot twice in a step). */
PKV_API int pkv_kv_append(const pkv_cache* cache, const void* k_new, const void* v_new,
                          int32_t in_dtype, int32_t n_tokens, const int32_t* slot_mapping,
                          const float* k_inv_scale, const float* v_inv_scale,
                          pkv_stream stream);

/* Slot mapping and KV append in one launch, for a batch (the same pages):
 * sequence s appends new tokens cu_new[s] … cu_new[s+1]−1 (rows of k_new /
 * v_new) at logical positions first_pos[s], first_pos[s]+1, …; each token's
 * slot is taken from the sequence's table row exactly as
 * pkv_slot_mapping_device computes it (−1 when the block is beyond max_blocks
 * or the entry is negative; such tokens are skipped), and stored values are
 * those of pkv_kv_append.
 *   cu_new:       device int32 [num_seqs + 1], nondecreasing, cu_new[0] = 0
 *   first_pos:    device int32 [num_seqs]
 *   max_new:      host bound on cu_new[s+1] − cu_new[s] (sizes the grid;
 *                 tokens past it are not appended)
 *   block_tables: device int32 [num_seqs, max_blocks]
 *   out_slots:    device int32 [cu_new[num_seqs]] receiving the slots, or NULL
 * Under PKV_CHECK=1 cu_new is copied back and checked against max_new. */
PKV_API int pkv_kv_append_paged(const pkv_cache* cache, const void* k_new, const void* v_new,
                                int32_t in_dtype, int32_t num_seqs, const int32_t* cu_new,
                                const int32_t* first_pos, int32_t max_new, const int32_t* block_tables,
                                int32_t max_blocks, const float* k_inv_scale, const float* v_inv_scale,
                                int32_t* out_slots, pkv_stream stream);

/* ---------------------------------------------------------------------------
 * Paged decode attention with split-KV — [P2] Q027 (online softmax: running
 * max m, sum l = Σ exp(s−m), weighted sum u = Σ exp(s−m)·v, output u/l, and
 * the merge that rescales old statistics by exp(m_old − m_new)); [P2] Q028
 * and [P3] 6.5 (the kernel reads K/V through the block table); [P1] formula
 * section and [P4] formula section (softmax(QKᵀ/√d + causal mask)·V).
 *
 * Each sequence b has one new query per head at logical position
 * seq_lens[b] − 1 and attends to all seq_lens[b] cached tokens (its own
 * just-appended K/V included). seq_lens[b] == 0 writes zeros.
 *   q:            device [batch, num_q_heads, head_dim] in q_dtype
 *                 (F32 for an F32 cache; BF16 for BF16 and FP8 caches)
 *   block_tables: device int32 [batch, max_blocks]
 *   seq_lens:     device int32 [batch]; values above max_seq_len are clamped
 *   max_seq_len:  host bound on seq_lens (sizes the grid and the workspace)
 *   scale:        score scale (1/sqrt(head_dim) for standard attention)
 *   partition_tokens: tokens per split-KV partition, a multiple of 16 in
 *                 [16, 8192] (a partition may end inside a 32- or 64-token
 *                 block); 0 picks one from the shape
 *                 (pkv_attn_decode_auto_partition)
 *   out:          device fp32 [batch, num_q_heads, head_dim], 16-byte aligned
 *   workspace:    device, 16-byte aligned, at least
 *                 pkv_attn_decode_workspace_bytes(...) bytes for the same
 *                 arguments; may be NULL when that size is 0 (a single
 *                 partition covers max_seq_len). It holds the partitions'
 *                 fp32 weighted sums u [batch, Hq, P, head_dim] followed by
 *                 their (m, l) pairs [batch, Hq, P, 2], P =
 *                 ceil(max_seq_len / partition). Its contents need no
 *                 initialisation; calls that share a workspace must not
 *                 overlap (one workspace per stream).
 * When more than one partition is needed the call launches two kernels on
 * the stream: the split kernel, then a small reduce kernel that merges the
 * partitions. BF16 and FP8 caches run the split on the matrix cores (the
 * query heads of a KV group are one side of 16×16 products), F32 caches on
 * the vector ALUs; see pkv_attn_decode_auto_partition for the override.
 * The result does not depend on the physical block ids: relabelling blocks
 * (with the same contents) gives bit-identical output.
 * num_q_heads must be a multiple of num_kv_heads with Hq/Hkv <= 64. */
PKV_API size_t pkv_attn_decode_workspace_bytes(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t head_dim,
                                               int32_t max_seq_len, int32_t partition_tokens);

PKV_API int pkv_attn_decode(const pkv_cache* cache, const void* q, int32_t q_dtype,
                            int32_t batch, int32_t num_q_heads, const int32_t* block_tables,
                            int32_t max_blocks, const int32_t* seq_lens, int32_t max_seq_len,
                            float scale, int32_t partition_tokens, float* out,
                            void* workspace, size_t workspace_bytes, pkv_stream stream);

/* pkv_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The split-KV partials go to the
 * library's own static device array of 8 MiB (8,388,608 bytes) per GPU,
 * which each GPU the library runs on holds until the process ends; its
 * device address is looked up on the first call on a device. The call
 * allocates nothing and launches the same kernels with the same partition
 * choice as pkv_attn_decode, so the output is identical. The caller passes
 * inputs and outputs as for pkv_attn_decode.
 * PKV_EWORKSPACE (nothing launched) if pkv_attn_decode_workspace_bytes for
 * the same arguments exceeds 8 MiB (for example batch 4, 32 query heads,
 * head_dim 128 and 64 partitions need 4.26 MB; pick larger partitions
 * otherwise). Every call on one GPU shares that GPU's array: calls that may
 * overlap on one GPU (several streams, several threads) race and must be
 * serialised by the caller. The array needs no clearing (its contents are
 * written before they are read in every call). PKV_CHECK is not honoured
 * here (its checking copies would allocate and synchronise). */
PKV_API int pkv_attn_decode_noalloc(const pkv_cache* cache, const void* q, int32_t q_dtype, int32_t batch,
                                    int32_t num_q_heads, const int32_t* block_tables, int32_t max_blocks,
                                    const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                    int32_t partition_tokens, float* out, pkv_stream stream);

/* The decode step's append and attention in one launch (BF16 and FP8
 * caches): sequence b's new token k_new[b], v_new[b] ([batch, num_kv_heads,
 * head_dim] in in_dtype, 16-byte aligned; BF16 for a BF16 cache, BF16 or F32
 * for an FP8 cache, which stores e4m3(x · inv_scale) as pkv_kv_append does)
 * is the token at position seq_lens[b] − 1 (its block already in the table;
 * [P2] Q025 and [P3] 6.1: append, then attend). The split kernel writes it to
 * that slot and attends to it from k_new / v_new, so the pool ends up as
 * after pkv_kv_append_paged and the output equals pkv_attn_decode's on that
 * pool. Other arguments as pkv_attn_decode. For an F32 cache, or with
 * PKV_DECODE_KERNEL=vector, the call runs an append launch and then the
 * decode. */
PKV_API int pkv_attn_decode_append(const pkv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                                   const float* k_inv_scale, const float* v_inv_scale, const void* q,
                                   int32_t q_dtype, int32_t batch, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                   int32_t max_seq_len, float scale, int32_t partition_tokens, float* out,
                                   void* workspace, size_t workspace_bytes, pkv_stream stream);

/* The partition size pkv_attn_decode uses when partition_tokens is 0 for a
 * cache of cache_dtype: with units = batch · num_kv_heads · (query-head
 * chunks per KV head), every sequence is split into ceil(256 / units)
 * partitions — one 8-wave workgroup per MI355X compute unit, no split when
 * the units already fill the chip — rounded up to 16 tokens, at least 256
 * tokens (or max_seq_len if shorter) and at most 8192. A chunk is up to 16
 * query heads of one KV head for BF16 and FP8 caches (the matrix-core
 * kernel) and the largest of 8, 4, 2, 1 dividing Hq/Hkv for F32 caches (the
 * vector kernel). The environment variable PKV_DECODE_KERNEL=vector or
 * =matrix, read at every call, selects the kernel for BF16 and FP8 caches
 * instead (for tests and tuning; F32 always uses the vector kernel). */
PKV_API int32_t pkv_attn_decode_auto_partition(int32_t cache_dtype, int32_t batch, int32_t num_q_heads,
                                               int32_t num_kv_heads, int32_t max_seq_len);

/* ---------------------------------------------------------------------------
 * Causal chunked prefill over a cached prefix — [P3] 6.6 (long prefills are
 * split into chunks so decodes are not starved); [P2] Q027 core answer and
 * FlashAttention section (tiles of query rows, scale and mask fused, scores
 * and probabilities kept on chip, the same exact result); [P2] Q025 table
 * row 2 (a position sees itself and everything before it).
 *
 * Sequence s has C_s = q_start[s+1] − q_start[s] new queries whose K/V are
 * already appended; with T_s = seq_lens[s] cached tokens in total, query i
 * sits at position T_s − C_s + i and attends to keys 0 … T_s − C_s + i.
 *   q:        device [q_start[num_seqs], num_q_heads, head_dim], BF16
 *   q_start:  device int32 [num_seqs + 1], nondecreasing, q_start[0] = 0
 *   seq_lens: device int32 [num_seqs], T_s >= C_s
 *   max_q_len: host bound on C_s (sizes the grid)
 *   scale:    score scale, positive and finite (1/sqrt(head_dim) for standard
 *             attention); anything else is PKV_EINVAL
 *   out:      device fp32, same shape as q
 * Cache dtype BF16, block_size 8, 16, 32 or 64; head_dim 64 or 128; Hq/Hkv 1, 2
 * or a multiple of 4 up to 64. No workspace is needed.
 * Two kernels compute it: a tile kernel (64 query rows of one KV group per
 * workgroup in four key streams sharing 32-key tiles through LDS, or 128
 * rows in two streams, or 256 in one), and the matrix-core decode kernel
 * with (query head, query) pairs as its 16 columns and the keys split across
 * its waves (tables of at most 8192 tokens). With rows = num_seqs ·
 * max_q_len · num_q_heads, the call takes the column form when rows < 128 ·
 * 64 (too few to give half the compute units a tile kernel workgroup), the
 * tile kernel with 256 rows per workgroup when rows ≥ 2 · 256 · 256 and
 * head_dim is 128 (two per compute unit), with 128 when rows ≥ 128 · 256
 * (one per unit), and with 64 otherwise; the environment variable
 * PKV_PREFILL_KERNEL=tiles (64 rows), =tiles128, =tiles256 (128 at head_dim
 * 64) or =columns, read at every call, forces one where it applies
 * (=tiles16: the earlier tile kernel, 16 query rows per wave). Pools of
 * 8-token blocks always take the tile kernel (64, 128 or 256 rows), whose
 * 16-row units then span table entries 2u and 2u+1. */
PKV_API int pkv_attn_prefill_chunk(const pkv_cache* cache, const void* q, int32_t q_dtype,
                                   int32_t num_seqs, int32_t num_q_heads, const int32_t* q_start,
                                   const int32_t* block_tables, int32_t max_blocks,
                                   const int32_t* seq_lens, int32_t max_q_len, float scale,
                                   float* out, pkv_stream stream);

/* ---------------------------------------------------------------------------
 * One continuous-batching step over a mixed batch — [P3] 6.6 (at an
 * iteration boundary some sequences run a prefill chunk while the others
 * decode one token; chunked prefill keeps long prompts from starving the
 * decodes); [P2] Q025 and [P3] 6.1 (append a token's K/V, then attend).
 *
 * The chunk sequences' new K/V are appended and their chunks attend causally
 * (as pkv_kv_append_paged followed by pkv_attn_prefill_chunk), and every
 * decode sequence appends its token and attends (as pkv_attn_decode_append).
 * By default, when the prefill takes the key-stream kernel's 64-row form on
 * blocks of 16 tokens or more, the decode partitions hold at most 4096
 * tokens and the decodes are large enough to run beside it (batch ·
 * max_seq_len · Hkv ≥ 2^20; PKV_MIXED=pair forces it), all of it is one
 * launch of four-wave workgroups, two per compute
 * unit: first the workgroups appending the chunks' tokens, then the chunks'
 * prefill query tiles (one per unit in the first round of dispatch), then
 * the decodes, which run beside them; a prefill wave waits on a per-call
 * counter for the appends only before it requests its first tile holding
 * chunk keys (a library-owned table of 1024 such counters per GPU, so at
 * most 1024 of these calls may be in flight on one GPU). The pool bytes are
 * bit-identical to the separate calls', the outputs equal theirs up to the
 * summation order (two key streams instead of four; four decode waves
 * instead of eight). When the prefill alone would take the column form
 * (small chunks): with fewer than 128 query blocks all of it is one launch of
 * the decode body (appends, decodes, then the query blocks, which wait for
 * the appends), bit-identical to the separate calls; with more, the paired
 * launch above where its conditions hold, its prefill on the key-stream
 * tiles (unless PKV_PREFILL_KERNEL names a kernel). Otherwise, or with the environment
 * variable PKV_MIXED=two, two launches: the decode kernel, whose last workgroups
 * write the chunks' tokens, then the prefill kernel; PKV_MIXED=one: one
 * launch of eight-wave workgroups (appends, decodes, then the prefill
 * waiting for the appends). Both are bit-identical to the separate calls in
 * pool bytes and outputs. In every form the split-KV reduce follows as a
 * launch of its own when the decodes use more than one partition.
 *   chunks:  see pkv_chunk_batch; num_seqs may be 0
 *   decodes: see pkv_decode_batch; batch may be 0
 * BF16 cache and inputs, block_size 8, 16, 32 or 64, the matrix-core decode whatever
 * PKV_DECODE_KERNEL says. A chunk's new positions must not lie in blocks the
 * decodes read (shared prefix blocks are full, so copy-on-write of a shared
 * tail keeps this). */
typedef struct pkv_chunk_batch {
  int32_t num_seqs;
  const void* q;                 /* as pkv_attn_prefill_chunk                    */
  const int32_t* q_start;
  const void* k_new;             /* device [q_start[num_seqs], Hkv, head_dim]:  */
  const void* v_new;             /*   rows of sequence s are its last C_s tokens */
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* seq_lens;       /* T_s, the chunk's tokens included           */
  int32_t max_q_len;
  float* out;
} pkv_chunk_batch;

typedef struct pkv_decode_batch {   /* as pkv_attn_decode_append              */
  int32_t batch;
  const void* q;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;
  int32_t max_blocks;               /* >= 1 even when batch is 0             */
  const int32_t* seq_lens;
  int32_t max_seq_len;
  int32_t partition_tokens;
  float* out;
  void* workspace;
  size_t workspace_bytes;
} pkv_decode_batch;

PKV_API int pkv_attn_mixed_step(const pkv_cache* cache, int32_t num_q_heads, float scale,
                                const pkv_chunk_batch* chunks, const pkv_decode_batch* decodes,
                                pkv_stream stream);

/* ---------------------------------------------------------------------------
 * Copy-on-write block copy — [P2] Q028 (sharing a partly filled last block
 * and then writing to it needs a copy, or one sequence's append corrupts the
 * other's; table row 6); [P3] 6.5 (copy-on-write with reference counts).
 * Copies whole blocks (K and V, every head): src[i] → dst[i].
 *   src, dst: device int32 [n]; ids outside the pool are skipped.
 * Destinations must be distinct and must not also be sources. */
PKV_API int pkv_copy_blocks(const pkv_cache* cache, const int32_t* src, const int32_t* dst,
                            int32_t n, pkv_stream stream);

/* ---------------------------------------------------------------------------
 * Swap blocks out to host memory and back — [P4] closing section, table of
 * the four remedies for a full cache, row "move it away for now" (KV not
 * needed for a while goes to CPU memory and comes back when needed, at the
 * cost of moving it); [P2] Q028 follow-up on what a server can do when
 * memory runs short (preempt requests and move their state elsewhere).
 * Whole blocks (K and V, every head) move between the pool and a pinned host
 * buffer laid out [n][K block bytes, V block bytes] (block bytes =
 * num_kv_heads · block_size · head_dim · element size).
 *   ids:  device int32 [n]; slot i holds block ids[i]. Ids outside the pool
 *         are skipped (their host slot, or nothing in the pool, is written).
 *   host: pinned host memory (hipHostMalloc, or a torch pin_memory tensor),
 *         16-byte aligned, at least host_bytes ≥ n · 2 · block bytes;
 *         anything else is rejected (PKV_EINVAL) before any launch.
 * Asynchronous on the stream; the host copy is complete once the stream is.
 * Swap-in destinations must be distinct. */
PKV_API int pkv_swap_out(const pkv_cache* cache, const int32_t* ids, int32_t n, void* host, size_t host_bytes,
                         pkv_stream stream);
PKV_API int pkv_swap_in(const pkv_cache* cache, const void* host, size_t host_bytes, const int32_t* ids, int32_t n,
                        pkv_stream stream);

/* Measurement aid (not on the attention path): the HBM read rate for the
 * access pattern of paged decode, which streams 4 KiB (block, head) tiles
 * found through a block table ([P2] Q028; [P3] 6.5). Reads tiles of 4096
 * bytes from buf in the order tile_ids gives, with the decode kernels'
 * non-temporal buffer loads, in num_workgroups workgroups of 8 waves:
 * workgroup i reads ids [i*n_tiles/num_workgroups, (i+1)*n_tiles/num_workgroups)
 * and writes the XOR of every dword it read to sink[i].
 *   buf: device, buf_tiles * 4096 bytes, 16-byte aligned; ids outside
 *        [0, buf_tiles) are skipped.
 *   tile_ids: device int32 [n_tiles]; sink: device uint32 [num_workgroups].
 * PKV_EINVAL for negative sizes, NULL pointers or a misaligned buf.
 * Asynchronous on the stream. */
PKV_API int pkv_debug_stream_read(const void* buf, int64_t buf_tiles, const int32_t* tile_ids, int32_t n_tiles,
                                  int32_t num_workgroups, uint32_t* sink, pkv_stream stream);

/* Measurement aid (not on the attention path): the bf16 matrix-core rate
 * the GPU sustains with every compute unit busy, for the products of the
 * chunked prefill's steady iteration ([P2] Q027, the FlashAttention section:
 * QK^T and PV done tile by tile on chip). Each of num_workgroups workgroups
 * of 8 waves issues, per wave and per iteration, the 24
 * v_mfma_f32_32x32x16_bf16 of that iteration in the same order and on the
 * same five accumulators (four PV, one QK^T), and nothing else.
 *   operands: device bf16, at least 8*(64+19) = 664 values, 16-byte aligned;
 *             lane l reads values [8(l+j), 8(l+j)+8) as operand j < 20.
 *   sink: device float [num_workgroups * 512]; lane l of wave w of workgroup
 *         g writes the sum of its accumulators' 80 values to
 *         sink[512 g + 64 w + l] (with every operand 1.0: 6144 * iterations).
 * Flops per call: num_workgroups * 8 * iterations * 24 * 2 * 32*32*16.
 * PKV_EINVAL for a negative iteration count, num_workgroups outside
 * [1, 2^31 - 1], NULL pointers or misaligned operands. Asynchronous. */
PKV_API int pkv_debug_mfma_rate(const void* operands, int32_t iterations, int32_t num_workgroups, float* sink,
                                pkv_stream stream);

/* Measurement aid: the chunked prefill's steady iteration with its data
 * movement and without its arithmetic dependences ("07｜KV Cache、
 * FlashAttention与PagedAttention的内部过程", FlashAttention section: tiles
 * staged on chip, products done tile by tile). Per wave and iteration: the
 * same 24 v_mfma_f32_32x32x16_bf16 products as pkv_debug_mfma_rate, 96
 * vector FMAs and 16 exponentials over the Sᵀ results; mode 1 adds the
 * prefill's LDS operand reads (8 ds_read_b128 of a K tile, 16 transposing
 * 8-byte reads of a V tile: 128 KiB per workgroup and iteration); mode 2 also
 * its tile stream (8 LDS-direct loads of 1 KiB per wave, 64 KiB per
 * workgroup), a wait for them and a workgroup barrier. One 8-wave workgroup
 * per num_workgroups entry, 128 KiB of LDS each.
 *   operands: device bf16, at least 664 values, 16-byte aligned;
 *   tiles: device, tiles_bytes ≥ 1 MiB (only the first MiB is read), 16-byte
 *          aligned: the first 64 KiB fill the LDS read region, the tile
 *          loads read 1 KiB units of the first MiB;
 *   sink: device fp32 [num_workgroups * 512], written.
 * Flops per call: num_workgroups * 8 * iterations * 24 * 2 * 32*32*16.
 * PKV_EINVAL for a negative iteration count, num_workgroups outside
 * [1, 2^31 - 1], a mode outside 0-2, tiles below 1 MiB, NULL pointers or
 * misaligned operands or tiles. Asynchronous. */
PKV_API int pkv_debug_prefill_mix(const void* operands, const void* tiles, int64_t tiles_bytes, int32_t mode,
                                  int32_t iterations, int32_t num_workgroups, float* sink, pkv_stream stream);

/* Test aid: read one sequence back through its table into the semantic
 * layout [num_kv_heads, seq_len, head_dim] of the stored dtype ([P2] Q025:
 * K and V each [B, H_kv, T, Dh]; Q028: paging changes placement, not order).
 *   block_table: device int32 [ceil(seq_len / block_size)]
 *   k_out, v_out: device, num_kv_heads*seq_len*head_dim stored elements. */
PKV_API int pkv_debug_gather(const pkv_cache* cache, const int32_t* block_table,
                             int32_t seq_len, void* k_out, void* v_out, pkv_stream stream);

/* ---------------------------------------------------------------------------
 * Host block allocator — [P2] Q028 core answer and follow-ups (allocate
 * blocks on demand, return them to the pool when released, share identical
 * prefixes with reference counts, copy-on-write for a shared partial tail);
 * [P3] 6.5 (the request flow); [P1] engine section (a finished request must
 * not free pages another request still uses). Never touches device memory.
 *
 * Single-threaded: calls on one allocator must not overlap. Every call is
 * all-or-nothing: on error the allocator state is unchanged. Free blocks form
 * a LIFO stack; the first allocations return free_order[0], free_order[1], …
 * (or 0, 1, 2, … when free_order is NULL). Only full blocks should be shared;
 * a shared partial tail is copied on the next append.
 * ------------------------------------------------------------------------- */
typedef struct pkv_alloc pkv_alloc;

/* free_order: host int32 [num_blocks], a permutation of 0..num_blocks−1, or NULL. */
PKV_API int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                             pkv_alloc** out);
PKV_API void pkv_alloc_destroy(pkv_alloc* a);

/* Take n blocks (refcount 1 each) into host out_ids[n]; PKV_ENOBLOCKS if
 * fewer than n are free. */
PKV_API int pkv_alloc_allocate(pkv_alloc* a, int32_t n, int32_t* out_ids);

/* Add one reference to each listed live block (sharing a prefix).
 * PKV_EINVAL for an id outside the pool, PKV_EREF for a free block. */
PKV_API int pkv_alloc_incref(pkv_alloc* a, const int32_t* ids, int32_t n);

/* Drop one reference per listing; a block returns to the pool at zero.
 * PKV_EREF if a block would drop below zero (duplicates count). */
PKV_API int pkv_alloc_decref(pkv_alloc* a, const int32_t* ids, int32_t n);

/* Reference count of a block (>= 0), or PKV_EINVAL. */
PKV_API int pkv_alloc_refcount(const pkv_alloc* a, int32_t id);
PKV_API int32_t pkv_alloc_num_free(const pkv_alloc* a);

/* Make the host block_table [max_blocks] of a sequence holding seq_len tokens
 * cover positions seq_len … seq_len+n_new−1: new blocks are allocated when a
 * position crosses into an unallocated block ([P2] Q028: positions 10 and 11
 * fill block 19, position 12 needs a new block), and a shared partially
 * filled tail is replaced by a private copy first. The copy is reported in
 * cow_src[0]/cow_dst[0] (host, capacity >= 1) with *n_cow = 1 (else 0); the
 * caller must run pkv_copy_blocks for it before appending.
 * PKV_EINVAL if the table would exceed max_blocks or holds an invalid id
 * within its first ceil(seq_len/bs) entries; PKV_ENOBLOCKS if the pool is short. */
PKV_API int pkv_alloc_reserve_append(pkv_alloc* a, int32_t* block_table, int32_t max_blocks,
                                     int32_t seq_len, int32_t n_new, int32_t* cow_src,
                                     int32_t* cow_dst, int32_t* n_cow);

/* ---------------------------------------------------------------------------
 * Prefix-cache index over full blocks — [P1] prefix-sharing section and its
 * token demo (cached ABCDEFGHIJKL vs new ABCDEFGXIJKL: reuse stops at the
 * first differing token and only whole pages count); [P1] engine section
 * (a full block's key chains its parent's key, its tokens and extra identity
 * such as model or adapter); [P3] 6.4 (chained hash of parent and block
 * tokens; a partial block is not reused; token hit rate = hit tokens /
 * compared prompt tokens; request hit rate = requests with any hit /
 * requests). Host only; single-threaded like the allocator.
 *
 * Keys are compared exactly (parent entry, identity and the block's tokens);
 * the chained 64-bit hash only selects candidates. When an allocator is
 * passed, each block the index takes on holds one reference until
 * pkv_prefix_clear, and each matched block gains one reference for the
 * caller; pass NULL to leave reference counts alone.
 * ------------------------------------------------------------------------- */
typedef struct pkv_prefix pkv_prefix;

/* block_size: tokens per block (the page) */
PKV_API int pkv_prefix_create(int32_t block_size, pkv_prefix** out);
PKV_API void pkv_prefix_destroy(pkv_prefix* idx);

/* Index the full blocks of host tokens[0..n_tokens): block i (i <
 * min(n_tokens / block_size, n_block_ids)) is held by block_ids[i]. A block
 * whose key is already indexed keeps its first id. *n_new (nullable)
 * receives how many blocks were newly indexed. All-or-nothing: with an
 * allocator, PKV_EREF (nothing indexed) if a new block is free. */
PKV_API int pkv_prefix_insert(pkv_prefix* idx, pkv_alloc* alloc, const int32_t* tokens, int32_t n_tokens,
                              uint64_t identity, const int32_t* block_ids, int32_t n_block_ids,
                              int32_t* n_new);

/* The longest run of indexed full blocks that starts the prompt host
 * tokens[0..n_tokens) under `identity`, stopping at the first block whose
 * key is not indexed, and at most max_ids blocks: their ids go to host
 * out_ids, their count to *n_match (so n_match·block_size prompt tokens need
 * no prefill). Counts one request, n_tokens compared tokens and
 * n_match·block_size hit tokens. */
PKV_API int pkv_prefix_match(pkv_prefix* idx, pkv_alloc* alloc, const int32_t* tokens, int32_t n_tokens,
                             uint64_t identity, int32_t* out_ids, int32_t max_ids, int32_t* n_match);

/* Hit counters since creation and the number of indexed blocks (each
 * pointer nullable). */
PKV_API int pkv_prefix_stats(const pkv_prefix* idx, int64_t* hit_tokens, int64_t* compared_tokens,
                             int64_t* requests, int64_t* hit_requests, int32_t* num_entries);

/* Forget every indexed block (the counters stay). The allocator the index
 * took references with must be passed to release them; PKV_EINVAL otherwise. */
PKV_API int pkv_prefix_clear(pkv_prefix* idx, pkv_alloc* alloc);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
