// Chunked prefill, key-stream form: the kernel body, shared by the prefill
// launch (prefill.hip) and the one-launch mixed step (decode.hip).
//
// Method: "07｜KV Cache、FlashAttention与PagedAttention的内部过程", Q027 core
// answer and the FlashAttention section (tiles with scores and probabilities
// kept on chip, online softmax); "06 KV Cache…" 6.6 (a chunk's queries see the
// cached prefix and the chunk's earlier tokens); Q025 table row 2 (the causal
// mask includes the diagonal).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pkv {

// Key-stream form (the tile kernel): a workgroup of eight waves, two per SIMD,
// owns 32·RG query rows (GW ≤ 4 heads of one KV group × 32·RG/GW queries),
// RG = 2, 4 or 8. Wave w takes row group w % RG (32 rows) of key stream
// w / RG: stream s of the NS = 8/RG streams scores the 32-key tiles s, s+NS,
// …, and the RG waves of a stream share each tile through LDS (with RG = 4 a
// tile feeds twice the products per byte loaded, with RG = 8 four times).
// Two waves per SIMD let one wave's vector work, waits and loads run while
// the other's products occupy the matrix core. (The mixed step's paired
// launch runs a four-wave form, NS = 2 and RG = 2 with rings capped at 80
// KiB, so that a decode workgroup fits on the same CU; it also passes a gate
// that each wave waits on before its first tile holding the chunk's own
// keys.) Per tile:
//   * K and V reach LDS through LDS-direct buffer loads (no registers): one
//     1 KiB load writes 16 bytes per lane in lane order, so a lane's global
//     address decides which chunk of which row lands where. The waves of a
//     stream load the tile's two 16-row units (RG/2 waves each; with 8-token
//     blocks a unit's two halves come from two table entries). Rows past
//     the last key the workgroup sees, and blocks outside the pool, read as
//     zeros (and their scores are masked). Unit addresses come from a per-lane table built
//     once per 32 tiles; the loads of a tile are spread between the products
//     of the iteration before the one that needs them. K and V have rings of
//     their own (three and two slots at Dh 128 with RG = 2: all of the CU's
//     160 KiB).
//   * Sᵀ = K·Qᵀ on v_mfma_f32_32x32x16_bf16 (32 keys × the wave's 32 rows),
//     K operands read 16 bytes per lane, chunks XOR-swizzled by row so the 16
//     lanes of a read meet 16 different bank groups.
//   * Oᵀ += Vᵀ·Pᵀ on the same instruction. The Vᵀ operand comes straight from
//     the row-major V tile through the transposing read ds_read_b64_tr_b16
//     (chunks swizzled for it); the Pᵀ operand is the Sᵀ accumulator's own
//     register order, so P needs no shuffle. P enters as a bf16 high part
//     (truncated) plus the bf16 rounding of the rest (two products), which
//     keeps the probabilities to ~16 bits.
//   * Online softmax per row in the log2 domain with a lazily moved base: the
//     exponent base may trail the row's running maximum by up to 2^8, so l
//     and O are rescaled (o = u / l is the same for any base) only when a
//     tile raises some row's maximum by more than that — in practice on the
//     first tiles only.
//   * Iteration j: the scores of tile j become P(j) while the matrix cores run
//     PV of tile j−1 and Sᵀ of tile j+1; then one barrier makes the next
//     tiles visible to every wave of each stream and frees the slots the
//     next iteration's loads go to.
// The streams' states are merged through LDS at the end.
namespace {

constexpr int kStreams = 4;            // key streams of a workgroup (a wave per row half each)
constexpr int kSRows = 64;             // query rows of a workgroup
constexpr int kSTile = 32;             // keys per tile
constexpr int kSBatch = 32;            // tiles whose table entries one VGPR holds (two per tile)
constexpr float kSlack = 8.0f;         // log2 units the exponent base may trail a row's maximum
// The steady iteration skips the row maximum: it exponentiates against the
// row's current base and falls back to the full update only if some lane's
// tile sum passes 2^64 (fp32 and bf16 keep their precision up to 2^127, so
// any base within 64 of the maximum is exact to use).
constexpr float kGuard = 18446744073709551616.0f;   // 2^64

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
typedef __attribute__((address_space(4))) const int32_t const_i32;

struct SArgs {
  const uint8_t* kc;
  const uint8_t* vc;
  const uint16_t* q;
  const int32_t* q_start;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;
  int num_blocks, hkv, hq, max_blocks, num_qtiles, num_chunks, gw;
  int unit_shift;   // log2(block_size / 16): a pool block holds 1, 2 or 4 16-row units (0 for 8-token blocks)
  float scale_log2;
};

// XOR swizzles of an LDS tile row's 16-byte chunks. K: the 16 lanes of an
// Sᵀ operand read take rows 0..15 at one chunk → 16 positions of a 256-byte
// bank window. V: a transposing read takes 4 consecutive rows × 4 chunks per
// 32 lanes → again 16 positions.
template <int DH>
__device__ __forceinline__ int swz_k(int r) { return DH == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int DH>
__device__ __forceinline__ int swz_v(int r) { return DH == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// LDS-direct loads of one 16-row unit: load i moves 16 bytes per lane from
// voffset[i] + 1024·i to LDS address lds + 1024·i + 16·lane (the instruction
// offset moves both addresses). M0 carries the LDS address, set once per
// unit; the compiler keeps nothing in M0 in this kernel (gfx9 LDS
// instructions do not read it).
__device__ __forceinline__ void lds_load_unit4(i32x4_t rsrc, const int* vo, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %4\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %0, %5, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen offset:3072 lds"
      :
      : "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(lds), "s"(rsrc)
      : "memory");
}
__device__ __forceinline__ void lds_load_unit2(i32x4_t rsrc, const int* vo, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %0, %3, 0 offen lds\n\t"
      "buffer_load_dwordx4 %1, %3, 0 offen offset:1024 lds"
      :
      : "v"(vo[0]), "v"(vo[1]), "s"(lds), "s"(rsrc)
      : "memory");
}
// one load of a unit: instruction offset 1024·I (sets M0 itself, so the
// loads of a unit can be spread between other instructions)
template <int I>
__device__ __forceinline__ void lds_load_one(i32x4_t rsrc, int vo, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %0, %2, 0 offen offset:%3 lds"
      :
      : "v"(vo), "s"(lds), "s"(rsrc), "n"(1024 * I)
      : "memory");
}
// vmcnt ≤ N: every load but the last N has landed
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// The loads above are invisible to the compiler's wait counting: these waits
// (ordered against every memory access) cover them.
__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) { return (uint32_t)(uintptr_t)(lds_u8*)(p); }

// Ring depths of a key stream's LDS tiles. K of tile t stays in K slot t % RK
// from its request until the end of the iteration that exponentiates tile t
// (a redo of that tile reads it again); V of tile t stays in V slot t % RV
// until PV(t) is done. With RK = RV + 1 the K and V of one pair of requests
// are both first needed RK − 2 iterations after they are issued. The deepest
// rings that fit 160 KiB of LDS, at most KMAX K slots.
template <int DH, int NS, int KMAX = 5>
struct StreamRings {
  static constexpr int TB = kSTile * DH * 2;
  static constexpr int fit = (160 * 1024 / (NS * TB) + 1) / 2;   // NS·(2RK − 1)·TB ≤ 160 KiB
  static constexpr int RK = fit > KMAX ? KMAX : fit;
  static constexpr int RV = RK - 1;
  static_assert(RK >= 3, "one iteration of cover at least");
};

// Row groups of 32 query rows per key stream: 2 (64 rows per workgroup, four
// streams), 4 (128 rows, two streams) or 8 (256 rows, one stream: no merge
// across streams). Each doubling halves the workgroup's tile stream per
// product; rings of three K slots keep the loop's unrolled period at six
// iterations.
template <int RG>
struct StreamShape {
  static_assert(RG == 2 || RG == 4 || RG == 8, "two, four or eight row groups per stream");
  static constexpr int NS = 8 / RG;           // key streams of the eight waves
  static constexpr int ROWS = 32 * RG;        // query rows of a workgroup
  static constexpr int KMAX = RG == 2 ? 5 : 3;
};

// LDS bytes the body uses (its argument `lds`, 1 KiB aligned)
template <int DH, int NS, int RG = 2, int KMAX = StreamShape<RG>::KMAX>
constexpr int stream_lds_bytes() {
  constexpr int TB = kSTile * DH * 2;
  using Rg = StreamRings<DH, NS, KMAX>;
  constexpr int KV = NS * (Rg::RK + Rg::RV) * TB;
  constexpr int MERGE = NS == 1 ? 0 : RG * NS * ((DH / 32) * 16 + 2) * kWave * 4;
  return KV > MERGE ? KV : MERGE;
}

// A condition a key stream waits for before it requests its first tile that
// holds one of the chunk's own keys (their K/V written by the same launch):
// none here; a mixed step's one-launch form passes its own.
struct NoGate {
  static constexpr bool kActive = false;
  __device__ void wait() const {}
};

// The kernel's work for logical workgroup L (see xcd_logical_index), on RG·NS
// waves (8; or 4, two streams of two row groups, for a workgroup that shares
// its CU with another) and stream_lds_bytes<DH, NS, RG, KMAX>() bytes of LDS
// at `lds`. B8: pools of 8-token blocks; a 16-row unit is then the rows of
// table entries 2u and 2u+1, and each of its loads reads from one of the two.
template <int DH, int NS, int RG = 2, bool B8 = false, int KMAX = StreamShape<RG>::KMAX, class Gate = NoGate>
__device__ __forceinline__ void prefill_stream_body(const SArgs& a, uint8_t* lds, uint32_t L,
                                                    const Gate& gate = Gate{}) {
  static_assert(NS == StreamShape<RG>::NS || (NS == 2 && RG == 2), "NS streams of RG row groups: 8 or 4 waves");
  constexpr int NW = RG * NS;                 // waves: (stream, row group)
  constexpr int RB = DH * 2;                  // bytes of one key row of one head
  constexpr int TB = kSTile * RB;             // bytes of one K or V tile
  constexpr int RK = StreamRings<DH, NS, KMAX>::RK;
  constexpr int RV = StreamRings<DH, NS, KMAX>::RV;
  constexpr int NDC = DH / 16;                // k-steps of Sᵀ
  constexpr int NDT = DH / 32;                // 32-row dh tiles of Oᵀ
  constexpr int CPR = RB / 16;                // 16-byte chunks per row
  constexpr int RPL = kWave / CPR;            // rows per 1 KiB load
  constexpr int LPU = kBlockSize / RPL;       // loads per 16-row unit
  constexpr int WPU = RG / 2;                 // waves loading one unit
  constexpr int LPW = LPU / WPU;              // a wave's loads per unit request
  constexpr int PAIR = 2 * LPW;               // a wave's loads of one (K, V) request pair
  static_assert(LPW >= 1, "every wave loads part of a unit");
  static_assert(stream_lds_bytes<DH, NS, RG, KMAX>() <= 160 * 1024, "LDS of a CU");
  static_assert((4 * NDT) % NS == 0, "output groups per stream");
  static_assert(!B8 || RPL <= kBlockSize / 2, "with 8-token blocks a load lies in one block");
  constexpr int VB = B8 ? 4 : 2;              // validity bits per tile: 8- or 16-key pieces
  constexpr int VFULL = (1 << VB) - 1;
  // lds: [stream][K slot] tiles, then [stream][V slot]; the merge reuses it

  // workgroup → (sequence, KV head, head chunk, query tile); query tiles run
  // longest first (a chunk's last tile sees the most keys)
  const int qtile = a.num_qtiles - 1 - (int)(L % a.num_qtiles);
  const int chunk = (L / a.num_qtiles) % a.num_chunks;
  const int g = (L / a.num_qtiles / a.num_chunks) % a.hkv;
  const int s = L / a.num_qtiles / a.num_chunks / a.hkv;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rg = w % RG, stream = w / RG;
  // the wave's part of each tile's loads: unit `unit` (rows 16·unit …), its
  // loads sub·LPW … sub·LPW + LPW − 1
  const int unit = rg / WPU, sub = rg % WPU;
  // The first batch of table entries (see the request table below), read
  // before the sequence's lengths arrive: it needs only the table's size, so
  // the entries' latency overlaps the lengths'. Units past the keys the
  // workgroup sees are dropped when the table is built.
  const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks;
  // table entry of unit u (B8: its first half; h = 1: its second half)
  auto unit_id = [&](int u, int h) -> int {
    const int x = B8 ? 2 * u + h : u >> a.unit_shift;
    const int e = x < a.max_blocks ? bt[x] : -1;
    return (unsigned)e < (unsigned)a.num_blocks ? e : -1;
  };
  auto batch_unit = [&](int b) { return 2 * (stream + NS * (b * kSBatch + (lane >> 1))) + (lane & 1); };
  auto batch_ids = [&](int b) -> int { return unit_id(batch_unit(b), 0); };
  auto batch_ids2 = [&](int b) -> int { return B8 ? unit_id(batch_unit(b), 1) : -1; };
  const int ids0 = batch_ids(0);
  const int ids0b = batch_ids2(0);
  const int q_lo = __builtin_amdgcn_readfirstlane(a.q_start[s]);
  const int C = __builtin_amdgcn_readfirstlane(a.q_start[s + 1]) - q_lo;
  const int T = __builtin_amdgcn_readfirstlane(
      min(a.seq_lens[s], B8 ? a.max_blocks * (kBlockSize / 2) : (a.max_blocks << a.unit_shift) * kBlockSize));
  const int QW = StreamShape<RG>::ROWS / a.gw;  // queries of the workgroup
  if (qtile * QW >= C || T <= 0) return;       // uniform over the workgroup
  const int base_pos = T - C;                  // position of query 0
  const int n = lane & 31, hg = lane >> 5;     // Sᵀ column (the lane's row) and lane half

  // the lane's row: workgroup row rg·32 + n
  const int R = rg * 32 + n;
  const int qi = qtile * QW + R % QW;
  const bool row_ok = qi < C;
  const int row_q = q_lo + (row_ok ? qi : 0);
  const int row_head = g * (a.hq / a.hkv) + chunk * a.gw + R / QW;
  const int row_pos = row_ok ? base_pos + qi : T - 1;
  const int first_pos = base_pos + qtile * QW;                     // smallest query position
  const int kend = min(T, base_pos + min(C, qtile * QW + QW));      // keys the workgroup sees
  const int ntiles = (kend + kSTile - 1) / kSTile;
  const int NT = (ntiles + NS - 1) / NS;       // iterations; a stream's last tile may lie past kend

  // Qᵀ operands: k-step dc, lane (n, hg): Q[row][16dc + 8hg .. +7]
  bf16x8_t qop[NDC];
  {
    const uint16_t* qp = a.q + ((size_t)row_q * a.hq + row_head) * DH + 8 * hg;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
      qop[dc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 16 * dc));
  }

  uint8_t* const kst = lds + stream * RK * TB;
  uint8_t* const vst = lds + NS * RK * TB + stream * RV * TB;

  // LDS-direct load i of the wave's 16-row unit: lane → row i·RPL + lane/CPR
  // of the unit, LDS chunk position lane % CPR holding the row's chunk
  // (position ^ swizzle)
  // (the load's instruction offset adds 1024·i; across loads the K swizzle
  // changes by 4i in the chunk index, the V swizzle not at all)
  const int koff0 = (lane / CPR) * RB + (((lane % CPR) ^ swz_k<DH>(lane / CPR)) << 4);
  const int voff0 = (lane / CPR) * RB + (((lane % CPR) ^ swz_v<DH>(lane / CPR)) << 4);
  static_assert(DH == 64 || DH == 128, "the swizzle steps above");
  const int unit_mask = (1 << a.unit_shift) - 1;
  // bytes of one (pool block, head)
  const size_t head_stride = B8 ? (size_t)(kBlockSize / 2) * RB : ((size_t)kBlockSize * RB) << a.unit_shift;
  const char* kbase = reinterpret_cast<const char*>(a.kc);
  const char* vbase = reinterpret_cast<const char*>(a.vc);

  // Request table of the stream's tiles, one entry per lane: batch b holds
  // units 2t and 2t+1 of tiles t = stream + NS·(32b + lane/2) (ids from
  // batch_ids above). An entry is the K address of its unit (low word; the
  // next 16 address bits and the unit's bytes before the workgroup's last
  // visible key in the other word). An id outside the pool, or a unit past
  // that key, has 0 bytes: its loads fill zeros. Requests read entries back
  // with lane reads, so no iteration waits on a memory load or spends scalar
  // work on addresses. With 8-token blocks a second table holds each unit's
  // second block, its address taken 8 rows back so that the loads' offsets
  // (rows 8-15 of the unit) and the byte count mean the same in both.
  uint32_t tl, th;        // entries of the batch holding the next K request
  uint32_t tl2 = 0, th2 = 0;
  uint64_t vmask;         // bit 2i+h: unit h of the batch's tile i holds keys (B8: its first 8 rows)
  uint64_t vmask2 = 0;    // B8: bit 2i+h: the second 8 rows of unit h of tile i hold keys
  auto make_table = [&](int b, int e, int e2) {
    const int u = batch_unit(b);
    const int in_range = max(0, min(kBlockSize, kend - u * kBlockSize));   // the unit's rows before kend
    const int rows = e < 0 ? 0 : in_range;
    const uint64_t addr = (uint64_t)(kbase + ((size_t)(e < 0 ? 0 : e) * a.hkv + g) * head_stride +
                                     (size_t)((B8 ? 0 : u & unit_mask) * kBlockSize) * RB);
    tl = (uint32_t)addr;
    th = ((uint32_t)(addr >> 32) & 0xffffu) | ((uint32_t)(rows * RB) << 16);
    vmask = __builtin_amdgcn_ballot_w64(rows > 0);
    if constexpr (B8) {
      const int rows2 = e2 < 0 ? 0 : in_range;
      const uint64_t addr2 = e2 < 0 ? (uint64_t)kbase
                                    : (uint64_t)(kbase + ((size_t)e2 * a.hkv + g) * head_stride) -
                                          (uint64_t)((kBlockSize / 2) * RB);
      tl2 = (uint32_t)addr2;
      th2 = ((uint32_t)(addr2 >> 32) & 0xffffu) | ((uint32_t)(rows2 * RB) << 16);
      vmask2 = __builtin_amdgcn_ballot_w64(rows2 > kBlockSize / 2);
    }
  };
  make_table(0, ids0, ids0b);
  int ids_nxt = NT > kSBatch ? batch_ids(1) : -1;     // ids of the batch after it
  int ids_nxt2 = NT > kSBatch ? batch_ids2(1) : -1;
  const uint64_t dv = (uint64_t)(vbase - kbase);      // V's unit lies this far from K's
  // validity bits of tile t (in the current batch), one per 16-key unit, or
  // with 8-token blocks one per 8 keys
  auto vbits = [&](int t) -> int {
    const int sh = 2 * (t & (kSBatch - 1));
    const int v0 = (int)(uint32_t)(vmask >> sh) & 3;
    if constexpr (!B8) {
      return v0;
    } else {
      const int v1 = (int)(uint32_t)(vmask2 >> sh) & 3;
      return (v0 & 1) | ((v1 & 1) << 1) | ((v0 & 2) << 1) | ((v1 & 2) << 2);
    }
  };
  struct Ent {
    uint32_t lo, hi, lo2, hi2;
  };
  // the wave's entry of tile t; after a batch's last tile the next batch
  // becomes current
  auto take_entry = [&](int t) -> Ent {
    const int ln = 2 * (t & (kSBatch - 1)) + unit;
    Ent e{(uint32_t)__builtin_amdgcn_readlane((int)tl, ln), (uint32_t)__builtin_amdgcn_readlane((int)th, ln), 0u, 0u};
    if constexpr (B8) {
      e.lo2 = (uint32_t)__builtin_amdgcn_readlane((int)tl2, ln);
      e.hi2 = (uint32_t)__builtin_amdgcn_readlane((int)th2, ln);
    }
    if (((t + 1) & (kSBatch - 1)) == 0 && t + 1 < NT) {
      const int b = (t + 1) / kSBatch;
      make_table(b, ids_nxt, ids_nxt2);
      ids_nxt = NT > (b + 1) * kSBatch ? batch_ids(b + 1) : -1;
      ids_nxt2 = NT > (b + 1) * kSBatch ? batch_ids2(b + 1) : -1;
    }
    return e;
  };
  // A request: the unit's buffer resource and the LDS address of its slot
  // (K of tile t in K slot t % RK, V in V slot t % RV), then its LPU loads.
  struct Req {
    int lo, hi, bytes;    // buffer resource words 0-2
    uint32_t d;
    int lo2, hi2, bytes2; // B8: the resource of the unit's second block
  };
  auto make_req = [&](Ent e, bool is_v, int t) -> Req {
    uint64_t addr = ((uint64_t)(e.hi & 0xffffu) << 32) | e.lo;
    if (is_v) addr += dv;
    const uint8_t* slot = is_v ? vst + (t % RV) * TB : kst + (t % RK) * TB;
    Req q{(int)(uint32_t)addr, (int)(uint32_t)(addr >> 32), (int)(e.hi >> 16),
          lds_addr(slot + unit * (kBlockSize * RB)), 0, 0, 0};
    if constexpr (B8) {
      uint64_t addr2 = ((uint64_t)(e.hi2 & 0xffffu) << 32) | e.lo2;
      if (is_v) addr2 += dv;
      q.lo2 = (int)(uint32_t)addr2;
      q.hi2 = (int)(uint32_t)(addr2 >> 32);
      q.bytes2 = (int)(e.hi2 >> 16);
    }
    return q;
  };
  // (the resource is assembled from scalar words here: a vector of them
  // carried across iterations may be given vector registers)
  auto issue_one = [&](bool is_v, const Req& q, int i) {
    // B8: loads of rows 8-15 of the unit read its second block
    const bool second = B8 && (sub * LPW + i) * RPL >= kBlockSize / 2;
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane(second ? q.lo2 : q.lo);
    r[1] = __builtin_amdgcn_readfirstlane(second ? q.hi2 : q.hi);
    r[2] = __builtin_amdgcn_readfirstlane(second ? q.bytes2 : q.bytes);
    r[3] = kBufferRsrcWord3;
    const uint32_t d = __builtin_amdgcn_readfirstlane(q.d);
    switch (sub * LPW + i) {
      case 0: lds_load_one<0>(r, is_v ? voff0 : koff0, d); break;
      case 1: lds_load_one<1>(r, is_v ? voff0 : koff0 ^ 64, d); break;
      case 2: lds_load_one<2>(r, is_v ? voff0 : koff0 ^ 128, d); break;
      default: lds_load_one<3>(r, is_v ? voff0 : koff0 ^ 192, d); break;
    }
  };
  auto issue_req = [&](bool is_v, const Req& q) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) issue_one(is_v, q, i);
  };

  // Vᵀ operand reads: lane (group G = lane/16, m = lane%16) of dh tile dt,
  // key step ks, half hh addresses row 16ks + 8hh + 4(G/2) + m/4, columns
  // 32dt + 16(G%2) + 4(m%4) … +3; as m/4 ≡ row (mod 4), the swizzle turns
  // chunk 4dt + c into 4(dt ^ r) + c
  const int vm = lane & 15, vG = lane >> 4;
  const int vrow0 = 4 * (vG >> 1) + (vm >> 2);
  const int vcc = 2 * (vG & 1) + ((vm & 3) >> 1);
  int vaddr[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const int r3 = DH == 128 ? (vm >> 2) : ((vrow0 >> 1) & 1);
    vaddr[dt] = vrow0 * RB + ((4 * (dt ^ r3) + vcc) << 4) + (vm & 1) * 8;
  }
  // K operand reads: row n, chunk 2dc + hg
  int kaddr[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) kaddr[dc] = n * RB + (((2 * dc + hg) ^ swz_k<DH>(n)) << 4);

  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16_t{};
  float m_run = -INFINITY;    // exponent base of the lane's row (log2 units)
  float l_run = 0.0f;         // this lane's part of the row sum
  const float c2 = a.scale_log2;

  auto vread = [&](const uint8_t* vb, int dt, int ks) -> bf16x8_t {
    const uint8_t* p = vb + vaddr[dt] + ks * 16 * RB;
    const bf16x4_t a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_u8*)p);
    const bf16x4_t a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_u8*)(p + 8 * RB));
    const uint2 u0 = __builtin_bit_cast(uint2, a0), u1 = __builtin_bit_cast(uint2, a1);
    return __builtin_bit_cast(bf16x8_t, make_uint4(u0.x, u0.y, u1.x, u1.y));
  };
  auto kread = [&](const uint8_t* kb, int dc) -> bf16x8_t {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kb + kaddr[dc]));
  };
  auto scores = [&](int j) -> f32x16_t {
    const uint8_t* kb = kst + (j % RK) * TB;
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kread(kb, dc), qop[dc], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);     // operands read one product ahead at most (registers)
    }
    return acc;
  };
  struct Pbits {
    bf16x8_t hi[2], lo[2];    // key steps 0, 1 (keys 0-15 and 16-31 of the tile)
  };
  auto pv = [&](int j, const Pbits& P) {
    const uint8_t* vb = vst + (j % RV) * TB;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8_t vv = vread(vb, dt, ks);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, P.hi[ks], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, P.lo[ks], o[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // bf16 pairs (−1, 0) and (0, −1) for the exact remainder p − trunc_bf16(p)
  // on v_dot2c_f32_bf16. Held in registers the compiler cannot see into: as
  // a folded inline constant the pair (−1, 0) reaches the instruction as the
  // fp32 pattern of −1.0, i.e. the pair (0, −1).
  uint32_t kNegOne0, kNegOne1;
  asm("s_mov_b32 %0, 0xbf80" : "=s"(kNegOne0));
  asm("s_mov_b32 %0, 0xbf800000" : "=s"(kNegOne1));
  // The full update of tile j: mask, row maximum, base moved when the maximum
  // passes it by more than kSlack (l rescaled here; *alpha is O's factor),
  // P as high and low bf16 parts. Returns whether any row of the wave moved.
  // keys the lane's row does not see (causal mask, inclusive) or that lie in
  // units outside the pool: −inf; only tiles reaching past the workgroup's
  // first query, or holding such a unit, need it
  auto mask_scores = [&](int j, f32x16_t& st, int valid_units) {
    const int key0 = (stream + NS * j) * kSTile;
    if (key0 + kSTile - 1 > first_pos || valid_units != VFULL) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // (register r holds key 8(r/4) + 4hg + r%4 of the tile: 16-key unit
        // r/8, 8-key piece r/4)
        const int key = key0 + 8 * (r >> 2) + 4 * hg + (r & 3);
        if (key > row_pos || !((valid_units >> (B8 ? r >> 2 : r >> 3)) & 1)) st[r] = -INFINITY;
      }
    }
  };
  // the row maximum of (masked) scores, in log2 units
  auto row_max = [&](const f32x16_t& st) -> float {
    float mx = st[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, st[r]);
    return pair_halves32(mx, MaxOp()) * c2;
  };
  auto softmax = [&](int j, f32x16_t st, int valid_units, Pbits& P, float* alpha) -> bool {
    mask_scores(j, st, valid_units);
    const float mx = row_max(st);
    const bool need = mx > m_run + kSlack;             // never while the row has seen nothing (−inf)
    const float moved_by = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - mx);
    *alpha = need ? moved_by : 1.0f;
    m_run = need ? mx : m_run;
    l_run *= *alpha;
    const float mb = m_run == -INFINITY ? 0.0f : m_run;
    float ps = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(fmaf(st[8 * ks + 2 * i], c2, -mb));
        const float p1 = fast_exp2(fmaf(st[8 * ks + 2 * i + 1], c2, -mb));
        ps += p0 + p1;
        asm volatile("" : "+v"(ps));    // summed here, so p0 and p1 die with their remainders
        hw[i] = __builtin_amdgcn_perm(__float_as_uint(p1), __float_as_uint(p0), 0x07060302u);
        const float r0 = dot2_bf16(hw[i], kNegOne0, p0);     // p0 − its truncated bf16, exactly
        const float r1 = dot2_bf16(hw[i], kNegOne1, p1);
        lw[i] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)r0, (__bf16)r1});
      }
      P.hi[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      P.lo[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    }
    l_run += ps;
    // keep P's computation in this iteration's block (the compiler would sink
    // it to the next PV, past the branches, away from the products it should
    // overlap with)
    asm volatile("" : : "v"(P.hi[0]), "v"(P.hi[1]), "v"(P.lo[0]), "v"(P.lo[1]));
    return __builtin_amdgcn_ballot_w64(need) != 0;
  };

  // ---- Load protocol ----
  // Iteration j exponentiates tile j (scores from iteration j−1), runs PV of
  // tile j−1 and Sᵀ of tile j+1. Its end waits for request pair j (K of tile
  // j+2, V of tile j); the barrier then frees K of tile j and V of tile j−1,
  // and iteration j+1 issues pair j+RK−2 (K of tile j+RK, V of tile j+RK−2)
  // into those slots, its loads spread between its products so the vector
  // memory path moves them while the matrix cores work. Requests past NT fill
  // zeros. vq: validity bits of the tiles whose K is requested (bits VB·i …
  // VB·i + VB − 1: tile j+i); ea, eb: entries of the next two V requests, which trail
  // K by two tiles.
  // The prologue requests K of tiles 0 and 1 and pairs 0 … RK−4, and
  // prepares pair RK−3 for iteration 0 to issue (as iteration j−1 prepares
  // pair j+RK−3 for iteration j).
  int vq = 0;
  Ent ea, eb;
  bool gated = !Gate::kActive;   // the gate's wait is behind this wave (or there is none)
  auto gate_tile = [&](int t) {  // before the wave's first request of a tile holding chunk keys
    if constexpr (Gate::kActive) {
      if (!gated && (stream + NS * t) * kSTile + kSTile - 1 >= base_pos) {
        gate.wait();
        gated = true;
      }
    }
  };
  {
    Ent e[RK - 1];
#pragma unroll
    for (int t = 0; t < RK - 1; ++t) {
      gate_tile(t);
      vq |= vbits(t) << (VB * (t + 1));         // as at iteration −1: bits VB·i … for tile i−1
      e[t] = take_entry(t);
      issue_req(false, make_req(e[t], false, t));
      if (t >= 2) issue_req(true, make_req(e[t - 2], true, t - 2));   // pairs 0 … RK−4
    }
    ea = e[RK - 3];
    eb = e[RK - 2];
  }
  // V of "tile −1" (the slot iteration 0's PV reads, with P = 0): zeros, so
  // the first iteration's products add nothing
  {
    uint8_t* zslot = vst + ((RV - 1) % RV) * TB + unit * (kBlockSize * RB) + sub * LPW * 16 * kWave;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      *reinterpret_cast<uint4*>(zslot + (i * kWave + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
  }
  wait_loads_but<LPW + (RK - 3) * PAIR>();    // K of tile 0
  __syncthreads();
  f32x16_t s_cur = scores(0);
  {
    // each row's exponent base: the maximum of its visible scores in tile 0
    // (a row that sees none of them keeps −inf; its first visible tile takes
    // the full update through the steady iteration's redo)
    f32x16_t st = s_cur;
    mask_scores(0, st, vq >> VB & VFULL);
    m_run = row_max(st);
  }
  wait_loads_but<(RK - 3) * PAIR>();          // K of tile 1
  wait_lds_reads();
  __syncthreads();
  Pbits p_prev;
  p_prev.hi[0] = p_prev.hi[1] = p_prev.lo[0] = p_prev.lo[1] = bf16x8_t{};

  // the requests iteration j+1 issues (prepared during iteration j)
  Req pend_k, pend_v;
  auto prepare_next = [&](int j) {
    pend_v = make_req(ea, true, j + RK - 2);
    const int t = j + RK;
    gate_tile(t);
    const int nb = vbits(t);
    const Ent e = take_entry(t);
    pend_k = make_req(e, false, t);
    vq = (vq >> VB) | (nb << (VB * (RK - 1)));
    ea = eb;
    eb = e;
  };
  auto end_of_iteration = [&]() {
    wait_loads_but<(RK - 3) * PAIR>();        // pair j: K of tile j+2, V of tile j
    wait_lds_reads();
    __syncthreads();
  };
  prepare_next(-1);
  // Iteration j, scheduled by hand: the wave issues P(j)'s vector work
  // between the products and requests LDS operands well before they are
  // used; scheduling barriers fence each step so the compiler keeps this
  // order. Iteration 0's PV multiplies a zero P with zeros; the last
  // iteration's Sᵀ scores a tile past NT (zeros) and is not used.
  auto body_steady = [&](int j) {
    const uint8_t* vb = vst + ((j + RV - 1) % RV) * TB;     // V of tile j−1
    const uint8_t* kb = kst + ((j + 1) % RK) * TB;          // K of tile j+1
    f32x16_t st = s_cur;
    const int vu = vq & VFULL;
    mask_scores(j, st, vu);
    // A row without a base (−inf: it has seen no key yet) exponentiates
    // against 2^100 below zero: a visible key overflows to +inf, which sends
    // the tile to the redo below, and masked keys stay 0 (no NaN is ever
    // made: the guard's comparison is not NaN-safe under -fno-honor-nans).
    const float mb = m_run == -INFINITY ? -0x1p100f : m_run;
    bf16x8_t v0[NDT], v1[NDT], kk[NDC];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) v0[dt] = vread(vb, dt, 0);
    __builtin_amdgcn_sched_barrier(0);

    // P(j), two probabilities per piece, one piece per three products
    uint32_t hw[8], lw[8];
    float ps = 0.0f;
    auto piece = [&](int i) {
      const float p0 = fast_exp2(fmaf(st[2 * i], c2, -mb));
      const float p1 = fast_exp2(fmaf(st[2 * i + 1], c2, -mb));
      ps += p0 + p1;
      hw[i] = __builtin_amdgcn_perm(__float_as_uint(p1), __float_as_uint(p0), 0x07060302u);
      const float r0 = dot2_bf16(hw[i], kNegOne0, p0);
      const float r1 = dot2_bf16(hw[i], kNegOne1, p1);
      lw[i] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)r0, (__bf16)r1});
      // computed here, between these products (the compiler would otherwise
      // sink it to the next iteration, its only use)
      asm volatile("" : : "v"(hw[i]), "v"(lw[i]), "v"(ps));
    };
    // The 24 (Dh 128) or 12 (Dh 64) products: PV(j−1) key step 0 (high, then
    // low parts, dh-tile chains alternating), then key step 1 alternating
    // with the single-chain Sᵀ(j+1). Step k runs product k, then piece k/3
    // when k % 3 == 0; LDS operands are read at least two products ahead.
    constexpr int NSTEP = 6 * NDT;
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int k = 0; k < NSTEP; ++k) {
      if (k < NDT) {
        o[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0[k], p_prev.hi[0], o[k], 0, 0, 0);
        v1[k] = vread(vb, k, 1);
      } else if (k < 2 * NDT) {
        const int dt = k - NDT;
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0[dt], p_prev.lo[0], o[dt], 0, 0, 0);
        kk[dt] = kread(kb, dt);
      } else if (k < 4 * NDT) {
        const int h = (k - 2 * NDT) >> 1;
        if (((k - 2 * NDT) & 1) == 0) {
          o[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[h], p_prev.hi[1], o[h], 0, 0, 0);
          kk[NDT + h] = kread(kb, NDT + h);
        } else {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[h], qop[h], acc, 0, 0, 0);
        }
      } else {
        const int h = (k - 4 * NDT) >> 1;
        if (((k - 4 * NDT) & 1) == 0)
          o[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1[h], p_prev.lo[1], o[h], 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk[NDT + h], qop[NDT + h], acc, 0, 0, 0);
      }
      if (k % 3 == 0 && k / 3 < 8) piece(k / 3);
      if (k >= 1 && k <= LPW) issue_one(true, pend_v, k - 1);
      if (k > LPW && k <= 2 * LPW) issue_one(false, pend_k, k - 1 - LPW);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = NSTEP / 3; i < 8; ++i) piece(i);    // Dh 64: fewer products than pieces
    const bool redo = __builtin_amdgcn_ballot_w64(!(ps <= kGuard)) != 0;
    l_run += redo ? 0.0f : ps;
    p_prev.hi[0] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    p_prev.hi[1] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[4], hw[5], hw[6], hw[7]));
    p_prev.lo[0] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    p_prev.lo[1] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[4], lw[5], lw[6], lw[7]));
    s_cur = acc;
    if (redo) {
      // a tile well above some row's base: P(j) again with the full update,
      // from scores recomputed out of K of tile j (still in its slot; O holds
      // PV(j−1) by now, in the old base)
      float alpha;
      if (softmax(j, scores(j), vu, p_prev, &alpha)) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      }
    }
    prepare_next(j);
    end_of_iteration();
  };
  {
    // The ring slots repeat every RK·RV iterations (RV = RK − 1, coprime):
    // unrolled by that period the slots' LDS offsets are constants that the
    // reads carry as immediates. Where the period is long, two iterations per
    // trip still spare the copies of the operands one iteration hands on.
    constexpr int U = RK * RV <= 6 ? RK * RV : 2;
    int j = 0;
    for (; j + U - 1 < NT; j += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) body_steady(j + u);
    }
    for (; j < NT; ++j) body_steady(j);
  }
  pv(NT - 1, p_prev);

  // ---- merge the streams: each wave writes its Oᵀ, m and l; the waves of a
  // row group then finish a quarter (NS = 4) or half (NS = 2) of its outputs;
  // a single stream's waves write their rows' outputs directly ----
  wait_all_loads();            // requests past the last tile still write their zeros
  wait_lds_reads();
  if constexpr (NS == 1) {
    const float l_row = pair_halves32(l_run, AddOp());
    const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;    // no valid key at all: zeros
    if (row_ok) {
      float* op = a.out + ((size_t)row_q * a.hq + row_head) * DH + 4 * hg;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(op + 32 * dt + 8 * q4) =
              make_float4(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv, o[dt][4 * q4 + 2] * inv,
                          o[dt][4 * q4 + 3] * inv);
    }
    return;
  }
  __syncthreads();
  // Oᵀ parts as [wave][dt][q4][lane] float4 (values 4q4 … 4q4+3 of a lane's
  // accumulator), so each store and each read moves 16 bytes per lane
  float4* mo = reinterpret_cast<float4*>(lds);
  float* ml = reinterpret_cast<float*>(mo + (size_t)NW * NDT * 4 * kWave);   // [wave][64][2] m, l
  const float l_row = pair_halves32(l_run, AddOp());
  {
    float4* my = mo + (size_t)w * NDT * 4 * kWave;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        my[(dt * 4 + q4) * kWave + lane] =
            make_float4(o[dt][4 * q4], o[dt][4 * q4 + 1], o[dt][4 * q4 + 2], o[dt][4 * q4 + 3]);
    ml[(w * kWave + lane) * 2 + 0] = m_run;
    ml[(w * kWave + lane) * 2 + 1] = l_row;
  }
  __syncthreads();
  float f[NS], mx = -INFINITY, lsum = 0.0f;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    f[k] = ml[((RG * k + rg) * kWave + lane) * 2];
    mx = fmaxf(mx, f[k]);
  }
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const float lk = ml[((RG * k + rg) * kWave + lane) * 2 + 1];
    f[k] = f[k] == -INFINITY ? 0.0f : fast_exp2(f[k] - mx);
    lsum += f[k] * lk;
  }
  const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;    // no valid key at all: zeros
  if (row_ok) {
    float* op = a.out + ((size_t)row_q * a.hq + row_head) * DH + 4 * hg;
    constexpr int G = 4 * NDT / NS;                       // 4-value groups of this wave
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      const int gi = stream * G + gg, dt = gi >> 2, q4 = gi & 3;
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const float4 x = mo[((size_t)(RG * k + rg) * NDT * 4 + dt * 4 + q4) * kWave + lane];
        v[0] += f[k] * x.x;
        v[1] += f[k] * x.y;
        v[2] += f[k] * x.z;
        v[3] += f[k] * x.w;
      }
      *reinterpret_cast<float4*>(op + 32 * dt + 8 * q4) = make_float4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    }
  }
}

// The kernel arguments of a prefill call.
// (rows: the workgroup's query rows, StreamShape<RG>::ROWS)
inline SArgs make_sargs(const PrefillParams& p, int rows = kSRows) {
  const int group = p.num_q_heads / p.cache.num_kv_heads;
  const int gw = group >= 4 ? 4 : group;
  SArgs a;
  a.kc = static_cast<const uint8_t*>(p.cache.k);
  a.vc = static_cast<const uint8_t*>(p.cache.v);
  a.q = static_cast<const uint16_t*>(p.q);
  a.q_start = p.q_start;
  a.block_tables = p.block_tables;
  a.seq_lens = p.seq_lens;
  a.out = p.out;
  a.num_blocks = p.cache.num_blocks;
  a.hkv = p.cache.num_kv_heads;
  a.hq = p.num_q_heads;
  a.max_blocks = p.max_blocks;
  a.gw = gw;
  a.num_chunks = group / gw;
  a.num_qtiles = (p.max_q_len + (rows / gw) - 1) / (rows / gw);
  a.unit_shift = p.cache.block_size > kBlockSize ? __builtin_ctz((unsigned)p.cache.block_size / kBlockSize) : 0;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  return a;
}

// workgroups of a prefill call
inline size_t stream_workgroups(const PrefillParams& p, const SArgs& a) {
  return (size_t)p.num_seqs * a.hkv * a.num_chunks * a.num_qtiles;
}

}  // namespace

}  // namespace pkv
