// Device helpers of the KV append, shared by the append kernels and the
// decode kernel that appends a step's tokens in the same launch.
//
// Paging arithmetic: "07｜KV Cache、FlashAttention与PagedAttention的内部过程",
// Q028 (block-size-4 table): position p → logical block p / bs, offset p % bs,
// physical block from the table; slot = physical · bs + offset.
#pragma once

#include "device_common.h"
#include "launch.h"

namespace pkv {

// Slot of logical position pos through one sequence's table row; −1 when the
// position's block is beyond max_blocks, its entry is negative, or the slot
// does not fit in int32 (a garbage entry must not wrap into the pool: the
// product is formed in 64 bits, and any slot the pool can hold is below 2^31).
__device__ __forceinline__ int slot_of(const int32_t* __restrict__ bt, int max_blocks, int pos, int bs) {
  const int lb = pos / bs;
  if (pos < 0 || lb >= max_blocks) return -1;
  const int phys = bt[lb];
  if (phys < 0) return -1;
  const int64_t slot = (int64_t)phys * bs + pos % bs;
  return slot <= (int64_t)INT32_MAX ? (int)slot : -1;
}

// One token's K and V rows into its slot: threads t0, t0+nt, … of the
// workgroup stride over 16-byte input chunks of K then V (copy, or e4m3
// quantise per head), kAppendBatch chunks per thread in flight at a time (a
// step's few tokens wait on memory latency, not bandwidth).
constexpr int kAppendBatch = 4;
template <int IN, int OUT>
__device__ __forceinline__ void append_token(const uint8_t* __restrict__ k_new,
                                             const uint8_t* __restrict__ v_new, int tok, int slot,
                                             uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                             int num_blocks, int hkv, int dh,
                                             const float* __restrict__ k_inv,
                                             const float* __restrict__ v_inv, int t0, int nt, int bs) {
  if (slot < 0 || slot >= num_blocks * bs) return;   // skipped token
  const int blk = slot / bs, off = slot % bs;
  constexpr int IN_B = IN == kF32 ? 4 : 2;
  constexpr int EPC = 16 / IN_B;                       // input elements per 16-byte chunk
  const int chunks_per_head = dh / EPC;
  const int chunks = hkv * chunks_per_head;
  for (int c0 = t0; c0 < 2 * chunks; c0 += kAppendBatch * nt) {
    uint4 x[kAppendBatch];
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {
      // past the token's last chunk a lane reloads that chunk (no branch
      // around the loads, so they are in flight together) and skips its store
      const int c = min(c0 + u * nt, 2 * chunks - 1);
      const bool is_v = c >= chunks;
      const int cc = is_v ? c - chunks : c;
      x[u] = *reinterpret_cast<const uint4*>((is_v ? v_new : k_new) + ((size_t)tok * chunks + cc) * EPC * IN_B);
    }
    // keeps the loads here rather than sunk into the conditional stores
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) asm volatile("" : "+v"(x[u].x), "+v"(x[u].y), "+v"(x[u].z), "+v"(x[u].w));
#pragma unroll
    for (int u = 0; u < kAppendBatch; ++u) {
      const int c = c0 + u * nt;
      if (c >= 2 * chunks) break;
      const bool is_v = c >= chunks;
      const int cc = is_v ? c - chunks : c;
      const int h = cc / chunks_per_head;
      const int e0 = (cc % chunks_per_head) * EPC;
      const size_t dst_elem = (((size_t)blk * hkv + h) * bs + off) * dh + e0;
      uint8_t* dst_base = is_v ? vc : kc;
      if constexpr (OUT != kFP8) {
        *reinterpret_cast<uint4*>(dst_base + dst_elem * IN_B) = x[u];
      } else {
        const float inv = (is_v ? v_inv : k_inv)[h];
        float f[EPC];
        if constexpr (IN == kBF16) {
          const uint32_t w[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
        } else {
          f[0] = __uint_as_float(x[u].x); f[1] = __uint_as_float(x[u].y);
          f[2] = __uint_as_float(x[u].z); f[3] = __uint_as_float(x[u].w);
        }
        uint32_t packed[EPC / 4];
#pragma unroll
        for (int i = 0; i < EPC / 4; ++i) {
          uint32_t b = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) b |= encode_e4m3(f[4 * i + j] * inv) << (8 * j);
          packed[i] = b;
        }
        uint8_t* dst = dst_base + dst_elem;
        if constexpr (EPC == 8) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
        } else {
          *reinterpret_cast<uint32_t*>(dst) = packed[0];
        }
      }
    }
  }
}

}  // namespace pkv
