// Paged decode attention with split-KV partitions, for gfx950.
//
// Method: "07｜KV Cache、FlashAttention与PagedAttention的内部过程", Q027 — per
// query the running maximum m, exponent sum l = Σ exp(s − m) and weighted sum
// u = Σ exp(s − m)·v give o = u / l; statistics gathered against different
// maxima are combined after rescaling by exp(m_part − m_total). Q028 / "06 KV
// Cache…" 6.5 — keys and values are read through the block table. Attention
// itself is softmax(q·Kᵀ·scale)·V over every cached token ("04. 注意力与 KV 缓存"
// formula section; "03. KV Cache…" formula section); decode's single query sits
// at the last position, so nothing is masked but the unused tail of the last
// block.
//
// Two forms of the split kernel compute the same thing. The vector form
// (below, any cache dtype; the only one for fp32 caches) does the products on
// the vector ALUs; the matrix-core form (further down, bf16 and fp8 caches)
// does them on MFMA with the query heads of a KV group as one side of 16×16
// products. Both share the partial format and the reduce kernel.
//
// Vector form: one workgroup (NW = 8 waves) owns (sequence b, KV head g, a
// chunk of HC query heads of that group, partition π of part_tokens tokens).
// Each wave streams the blocks w, w+8, w+16, … of π in a single pass:
//   * the wave's block-table entries are loaded once, one per lane, and read
//     back with a lane read into a scalar register;
//   * K and V of the next block are loaded while the current one is used,
//     through raw buffer loads whose record limit masks what must not be read
//     (non-temporal: every byte is read once);
//   * K is held with few lanes per token row (LPK), so a score is a short DPP
//     sum and each lane computes few exponentials; V is held with a row per
//     RB/16 consecutive lanes (every load covers whole rows) and p moves from
//     the K lanes to the V lanes through a small per-wave LDS slot;
//   * online softmax per head in the log2 domain: the running max moves only
//     when a block raises it, and only then are l and the accumulators
//     rescaled (the wave-uniform branch is rarely taken once the max settles).
// At the end the wave's accumulators are summed over its lane groups, the
// waves are merged through LDS, and either o = u / l is written (one
// partition) or (m, l, u) go to the workspace for a second, small kernel that
// merges the partitions. (Merging in the last workgroup to finish would need
// a device-scope release per workgroup, which writes back the L2 of its XCD
// every time; the kernel boundary does that once.)
// Masked slots (past the sequence end) are selected out or read as zeros,
// never multiplied by zero, and blocks whose id is outside the pool are
// skipped: pool slots may hold NaN.
#include <atomic>
#include <mutex>

#include "append_common.h"
#include "device_common.h"
#include "launch.h"
#include "prefill_stream.h"

namespace pkv {

namespace {

constexpr int kMergeThreads = 256;


// Register layouts of one (block, head) tile of 16 token rows, RB bytes each.
// K: a row is read by LPK lanes (4, 8 or 16); lane (tk = lane / LPK,
//    jk = lane % LPK) holds rows tk + TPK·i (i < NTK) and, of each, the 16-byte
//    chunks c·LPK + jk (c < NCK). A score is a sum over the LPK lanes of a row.
// V: a row is read by LPV = RB/16 consecutive lanes, so each load covers whole
//    rows; lane (rv, cv) holds rows rv + RPV·i (i < NIV), bytes cv·16 … +15.
template <int KV, int DH, int LPK_>
struct Geometry {
  static constexpr int ESZ = KV == kF32 ? 4 : KV == kBF16 ? 2 : 1;  // stored bytes per element
  static constexpr int RB = DH * ESZ;         // bytes of one token row of one head
  static constexpr int EPC = 16 / ESZ;        // elements in a 16-byte slice
  // q dwords per 16-byte K slice: fp32 values, or packed bf16 pairs
  static constexpr int QD = KV == kF32 ? 4 : EPC / 2;
  static constexpr int LPK = LPK_ < RB / 16 ? LPK_ : RB / 16;
  static constexpr int TPK = kWave / LPK;     // rows per K load
  static constexpr int NTK = kBlockSize / TPK;
  static constexpr int NCK = RB / (16 * LPK);
  static constexpr int LPV = RB / 16;
  static constexpr int RPV = kWave / LPV;
  static constexpr int NIV = kBlockSize / RPV;
  static_assert(LPK >= 4 && NTK >= 1 && NCK >= 1 && LPV >= 4 && LPV <= 32 && NIV >= 1,
                "unsupported row size");
};

struct KernelArgs {
  uint8_t* kc;         // pools: read, and written only by the fused append
  uint8_t* vc;
  const float* k_scale;
  const float* v_scale;
  const void* q;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;
  float* ws_ml;
  float* ws_u;
  int num_blocks, hkv, hq, max_blocks, max_seq_len, part_tokens, num_parts, num_chunks;
  float scale_log2;  // scale · log2(e)
  // the fused append (matrix-core form): each sequence's new token
  const uint8_t* k_new;
  const uint8_t* v_new;
  const float* k_inv;
  const float* v_inv;
  int new_dtype;
  int block_size;    // pool block: 8, 16, 32 or 64 tokens (the matrix-core form; 16 for the vector form)
  // Further appends done by the last x_wgs workgroups of the matrix-core
  // form, kExtraTokens tokens each (a mixed step's prefill chunks): sequence
  // s's rows x_cu[s] … x_cu[s+1]−1 of x_k / x_v (new_dtype) are its last
  // C_s = x_cu[s+1] − x_cu[s] positions, x_lens[s] − C_s …, placed through
  // row s of x_tables.
  const uint8_t* x_k;
  const uint8_t* x_v;
  const int32_t* x_cu;
  const int32_t* x_lens;
  const int32_t* x_tables;
  int x_max_blocks, x_seqs, x_wgs_per_seq, x_wgs;
  // Chunked prefill on the matrix-core form: the 16 columns of a workgroup
  // are (query head, query) pairs, 2^p_hg_shift heads × 16 / 2^p_hg_shift
  // consecutive queries of one sequence; p_nqb query blocks per (sequence,
  // KV head, head chunk); q_start as in the prefill call.
  const int32_t* q_start;
  int p_hg_shift, p_nqb;
};

struct MergeArgs {
  const float* ws_ml;
  const float* ws_u;
  float* out;
  int num_parts;
};

// Workgroups that stay together on one XCD: the head chunks and partitions
// of up to four KV heads of one sequence (four when Hkv allows, else two or
// one). Keeping a sequence's neighbouring heads together keeps its pool
// blocks' adjacent head tiles on one XCD, and dealing the groups out in turn
// keeps a run of long sequences in a batch off any single XCD. (Measured: a
// contiguous range of sequences per XCD made a batch whose last 15 sequences
// were its longest 20% slower; single KV heads per XCD cost 1-2% on equal
// lengths.)
__device__ __forceinline__ uint32_t decode_xcd_group(const KernelArgs& a) {
  const int hg = a.hkv % 4 == 0 ? 4 : a.hkv % 2 == 0 ? 2 : 1;
  return (uint32_t)(a.num_chunks * a.num_parts * hg);
}

// Sum over groups of N consecutive lanes (N = 4, 8, 16 or 32); every lane
// of a group receives the same bits (each step adds a commutative pair).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f32<kQuadXor1>(x);
  x += dpp_f32<kQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kRowMirror>(x);
  if constexpr (N >= 32) x = pair_rows16(x, AddOp());
  return x;
}

// Combine x across the 64 / N lane groups of size N, keeping each lane's
// position within its group (row rotations by 4 and 8 lanes, then exchanges
// across rows); every lane receives the combination of its position's
// values. The order of combination may differ between lanes, so a sum may
// differ in its last bits from lane to lane; a max does not.
template <int N, typename Op>
__device__ __forceinline__ float across_groups(float x, Op op) {
  if constexpr (N <= 4) x = op(x, dpp_f32<kRowRor4>(x));
  if constexpr (N <= 8) x = op(x, dpp_f32<kRowRor8>(x));
  if constexpr (N <= 16) x = pair_rows16(x, op);
  return pair_halves32(x, op);
}


// Score contribution of one 16-byte K slice against one head's q slice.
template <int KV, int QD>
__device__ __forceinline__ float slice_dot(const uint32_t (&qs)[QD], const uint32_t (&k)[QD], float acc) {
  if constexpr (KV == kF32) {
#pragma unroll
    for (int i = 0; i < QD; ++i) acc = fmaf(__uint_as_float(qs[i]), __uint_as_float(k[i]), acc);
  } else {
#pragma unroll
    for (int i = 0; i < QD; ++i) acc = dot2_bf16(qs[i], k[i], acc);
  }
  return acc;
}

// A K slice as QD dwords in the q register format (fp8 → bf16 pairs, exact).
template <int KV, int QD>
__device__ __forceinline__ void k_operand(const uint4& x, uint32_t (&k)[QD]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  if constexpr (KV == kFP8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[2 * i] = fp8x2_to_bf16x2<false>(w[i]);
      k[2 * i + 1] = fp8x2_to_bf16x2<true>(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = w[i];
  }
}

// The EPC fp32 values of one 16-byte V slice.
template <int KV, int EPC>
__device__ __forceinline__ void slice_values(const uint4& v, float (&f)[EPC]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (KV == kF32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (KV == kBF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(w[i]); f[2 * i + 1] = bf16_hi(w[i]); }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2_t a = fp8x2_to_f32x2<false>(w[i]);
      const f32x2_t b = fp8x2_to_f32x2<true>(w[i]);
      f[4 * i] = a[0]; f[4 * i + 1] = a[1]; f[4 * i + 2] = b[0]; f[4 * i + 3] = b[1];
    }
  }
}

// exp2(m − mt), taken as 0 for an empty part (m = −inf), also when mt is −inf.
__device__ __forceinline__ float part_weight(float m, float mt) {
  return m == -INFINITY ? 0.0f : fast_exp2(m - mt);
}

// Order the compiler's LDS accesses of one wave around a lane exchange (the
// hardware already executes one wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int KV, int DH, int HC, int LPK_, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_split_kernel(KernelArgs a) {
  constexpr int kWaves = NW, kThreads = NW * kWave;
  using G = Geometry<KV, DH, LPK_>;
  constexpr int EPC = G::EPC, QD = G::QD, LPK = G::LPK, TPK = G::TPK, NTK = G::NTK, NCK = G::NCK;
  constexpr int LPV = G::LPV, RPV = G::RPV, NIV = G::NIV;
  constexpr bool kSameLayout = LPK == LPV;    // p is already in the lanes that hold V
  __shared__ float sh_u[kWaves][HC][DH];
  __shared__ float sh_m[kWaves][HC];
  __shared__ float sh_l[kWaves][HC];
  __shared__ __attribute__((aligned(16))) float sh_p[kWaves][kBlockSize][HC];   // K lanes → V lanes

  // ---- which (b, g, chunk, partition) ----------------------------------------
  const uint32_t L = grouped_xcd_index(flat_block_id(), flat_grid_size(), decode_xcd_group(a));
  const int chunk = L % a.num_chunks;
  const int part = (L / a.num_chunks) % a.num_parts;
  const int g = (L / a.num_chunks / a.num_parts) % a.hkv;
  const int b = L / a.num_chunks / a.num_parts / a.hkv;
  const int group = a.hq / a.hkv;
  const int h0 = g * group + chunk * HC;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  // the wave index, read from the first lane so that the compiler knows it is
  // wave-uniform (block ids and buffer resources derived from it stay scalar)
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int P = a.num_parts;
  const int tok0 = part * a.part_tokens;
  const size_t head_stride = (size_t)kBlockSize * G::RB;     // bytes of one (block, head)
  // Issued together with the length load rather than after it: the table
  // entries the partition can hold (one per lane; entries past the sequence
  // are masked once the length arrives).
  const int lb0 = tok0 / kBlockSize;
  const int cap = min(a.part_tokens / kBlockSize, a.max_blocks - lb0);   // blocks the partition can hold
  const int cap_w = cap > w ? (cap - w + kWaves - 1) / kWaves : 0;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + lb0;
  const int phys_all = lane < cap_w ? bt[w + kWaves * lane] : -1;
  const int seq_len = a.seq_lens[b];
  int ntok = 0;        // tokens of this partition, set once the length is known
  int my_phys = -1;     // the wave's table entries, masked to the sequence
  float sc = 0.0f;

  float m[HC], l[HC], acc[HC][EPC];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;
  }

  const int tk = lane / LPK, jk = lane % LPK;                 // K layout
  const int rv = lane / LPV, cv = lane % LPV;                 // V layout
  const int koff = tk * G::RB + jk * 16;
  const int voff = rv * G::RB + cv * 16;

  // q slices matching the lane's K chunks
  uint32_t qreg[HC][NCK][QD];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const size_t row = (size_t)b * a.hq + h0 + h;
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      const int e0 = (c * LPK + jk) * EPC;   // first element of the chunk
      if constexpr (KV == kF32) {
        const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.q) + row * DH + e0);
        qreg[h][c][0] = x.x; qreg[h][c][1] = x.y; qreg[h][c][2] = x.z; qreg[h][c][3] = x.w;
      } else {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + row * DH + e0;
#pragma unroll
        for (int k = 0; k < QD / 4; ++k) {
          const uint4 x = *reinterpret_cast<const uint4*>(qp + 8 * k);
          qreg[h][c][4 * k] = x.x; qreg[h][c][4 * k + 1] = x.y;
          qreg[h][c][4 * k + 2] = x.z; qreg[h][c][4 * k + 3] = x.w;
        }
      }
    }
  }
  // Buffer resources over the wave's j-th (block, head) tile of K and V. The
  // record limit is the block's valid rows: an id outside the pool, j past the
  // wave's last block and rows past the sequence end read as zeros without a
  // memory access, so loads need no branch and masked V rows are exact zeros.
  auto tile_rsrc = [&](const uint8_t* pool, int phys, int rows) {
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const uint8_t* base = pool + ((size_t)(ok ? phys : 0) * a.hkv + g) * head_stride;
    // the record count is wave-uniform; reading it from the first lane keeps
    // the resource in scalar registers (no per-lane loop around the loads)
    const int records = __builtin_amdgcn_readfirstlane(ok ? rows * G::RB : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, records, kBufferRsrcWord3);
  };
  auto rows_of = [&](int j) {   // valid rows of the wave's j-th block (wave-uniform)
    return min(kBlockSize, max(0, ntok - (w + kWaves * j) * kBlockSize));
  };
  auto load_block = [&](int j, uint4 (&kb)[NTK][NCK], uint4 (&vb)[NIV]) {
    const int phys = __builtin_amdgcn_readlane(my_phys, j);
    const int rows = rows_of(j);
    const auto rk = tile_rsrc(a.kc, phys, rows);
    const auto rvs = tile_rsrc(a.vc, phys, rows);
#pragma unroll
    for (int i = 0; i < NTK; ++i)
#pragma unroll
      for (int c = 0; c < NCK; ++c) kb[i][c] = buffer_load16_stream(rk, koff + i * TPK * G::RB + c * LPK * 16);
#pragma unroll
    for (int i = 0; i < NIV; ++i) vb[i] = buffer_load16_stream(rvs, voff + i * RPV * G::RB);
  };

  auto use_block = [&](int j, const uint4 (&kb)[NTK][NCK], const uint4 (&vb)[NIV]) {
    const int phys = __builtin_amdgcn_readlane(my_phys, j);
    if ((unsigned)phys >= (unsigned)a.num_blocks) return;     // contributes nothing
    const int rows = rows_of(j);                               // >= 1
    // scores of the lane's NTK rows for the HC heads (rows past the end: −inf)
    float s[HC][NTK];
#pragma unroll
    for (int i = 0; i < NTK; ++i) {
      float ps[HC];
#pragma unroll
      for (int h = 0; h < HC; ++h) ps[h] = 0.0f;
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        uint32_t kk[QD];
        k_operand<KV, QD>(kb[i][c], kk);
#pragma unroll
        for (int h = 0; h < HC; ++h) ps[h] = slice_dot<KV, QD>(qreg[h][c], kk, ps[h]);
      }
      const bool ok = tk + TPK * i < rows;
#pragma unroll
      for (int h = 0; h < HC; ++h) {
        const float v = group_sum<LPK>(ps[h]) * sc;
        s[h][i] = ok ? v : -INFINITY;
      }
    }
    // block max per head; rescale only when it raises the running max
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      float bm = s[h][0];
#pragma unroll
      for (int i = 1; i < NTK; ++i) bm = fmaxf(bm, s[h][i]);
      bm = across_groups<LPK>(bm, MaxOp());
      if (bm > m[h]) {
        const float alpha = m[h] == -INFINITY ? 0.0f : fast_exp2(m[h] - bm);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha;
        m[h] = bm;
      }
    }
    // p = 2^(s − m); every lane of a K row holds the same p, so l is summed
    // across K rows only at the end
    float p[HC][NTK];
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int i = 0; i < NTK; ++i) {
        p[h][i] = fast_exp2(s[h][i] - m[h]);
        l[h] += p[h][i];
      }
    // p of the lane's V rows
    float pv[HC][NIV];
    if constexpr (kSameLayout) {
#pragma unroll
      for (int h = 0; h < HC; ++h)
#pragma unroll
        for (int i = 0; i < NIV; ++i) pv[h][i] = p[h][i];
    } else {
      // the LPK lanes of a K row share out the heads; the wave's own slot of
      // sh_p is written and read back by that wave only
#pragma unroll
      for (int i = 0; i < NTK; ++i)
#pragma unroll
        for (int h = 0; h < HC; ++h)
          if (h % LPK == jk) sh_p[w][tk + TPK * i][h] = p[h][i];
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < NIV; ++i) {
        const float* src = sh_p[w][rv + RPV * i];
        if constexpr (HC % 4 == 0) {
#pragma unroll
          for (int h4 = 0; h4 < HC; h4 += 4) {
            const float4 x = *reinterpret_cast<const float4*>(src + h4);
            pv[h4][i] = x.x; pv[h4 + 1][i] = x.y; pv[h4 + 2][i] = x.z; pv[h4 + 3][i] = x.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < HC; ++h) pv[h][i] = src[h];
        }
      }
      wave_lds_sync();
    }
    // acc += p · v (V rows past the end were read as zeros)
#pragma unroll
    for (int i = 0; i < NIV; ++i) {
      float f[EPC];
      slice_values<KV, EPC>(vb[i], f);
#pragma unroll
      for (int h = 0; h < HC; ++h)
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(pv[h][i], f[e], acc[h][e]);
    }
  };

  // Partitions past the sequence end (and every partition of an empty
  // sequence) run through with no blocks: they leave m = −inf, l = 0 and u = 0,
  // which the reduce kernel weighs 0 (or, with one partition, an output of 0).
  // No early exit keeps the table load ahead of the length on every path.
  const int T = __builtin_amdgcn_readfirstlane(min(max(seq_len, 0), min(a.max_seq_len, a.max_blocks * kBlockSize)));
  ntok = min(a.part_tokens, T - tok0);
  const int nblk = ntok > 0 ? (ntok + kBlockSize - 1) / kBlockSize : 0;
  const int nbw = nblk > w ? (nblk - w + kWaves - 1) / kWaves : 0;   // this wave's blocks
  my_phys = lane < nbw ? phys_all : -1;
  sc = a.scale_log2;
  if constexpr (KV == kFP8) sc *= a.k_scale[g];

  uint4 k0[NTK][NCK], v0[NIV], k1[NTK][NCK], v1[NIV];
  load_block(0, k0, v0);
  {
    for (int j = 0; j < nbw; j += 2) {
      load_block(j + 1, k1, v1);
      use_block(j, k0, v0);
      load_block(j + 2, k0, v0);
      if (j + 1 < nbw) use_block(j + 1, k1, v1);
    }
  }

  // ---- the wave's totals -----------------------------------------------------------
  // l: one copy per K row group → combine across K row groups; acc: combine
  // across V row groups. Afterwards every lane holds the wave's totals.
#pragma unroll
  for (int h = 0; h < HC; ++h) l[h] = across_groups<LPK>(l[h], AddOp());
#pragma unroll
  for (int h = 0; h < HC; ++h)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = across_groups<LPV>(acc[h][e], AddOp());
  if (rv == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) sh_u[w][h][cv * EPC + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h) { sh_m[w][h] = m[h]; sh_l[w][h] = l[h]; }
  }
  __syncthreads();

  // ---- merge the waves ---------------------------------------------------------------
  const float vscale = KV == kFP8 ? a.v_scale[g] : 1.0f;
  for (int i = tid; i < HC * DH; i += kThreads) {
    const int h = i / DH, d = i % DH;
    float mt = sh_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mt = fmaxf(mt, sh_m[ww][h]);
    float u = 0.0f, lt = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float wt = part_weight(sh_m[ww][h], mt);
      u = fmaf(wt, sh_u[ww][h][d], u);
      lt = fmaf(wt, sh_l[ww][h], lt);
    }
    if (P == 1) {
      a.out[((size_t)b * a.hq + h0 + h) * DH + d] = lt > 0.0f ? u * vscale / lt : 0.0f;
    } else {   // partials for the reduce kernel
      a.ws_u[(((size_t)b * a.hq + h0 + h) * P + part) * DH + d] = u * vscale;
      if (d == 0) {
        float* ml = a.ws_ml + (((size_t)b * a.hq + h0 + h) * P + part) * 2;
        ml[0] = mt;
        ml[1] = lt;
      }
    }
  }
}

// Split-KV reduce: one workgroup per (sequence, query head) row. Partition
// π left m_π (log2 domain), l_π and u_π — an empty partition left m = −inf,
// l = 0 and an unwritten u, which gets weight 0 and is never read into the
// sum; with m* = max m_π the output is Σ 2^(m_π − m*) u_π / Σ 2^(m_π − m*) l_π
// (0 for a sequence with no tokens). Thread (d4, pg) merges, online, the
// columns 4·d4 … 4·d4+3 of partitions pg, pg + NG, … (four partitions per
// round, their loads in flight together); the NG groups are then combined
// through LDS in a fixed order.
template <int DH>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(MergeArgs a) {
  constexpr int D4 = DH / 4, NG = kMergeThreads / D4;
  __shared__ float s_m[NG], s_l[NG];
  __shared__ float4 s_u[NG][D4];
  const size_t row = blockIdx.x;
  const int t = threadIdx.x, d4 = t % D4, pg = t / D4;
  const int P = a.num_parts;
  const float* ml = a.ws_ml + row * P * 2;
  const float4* u = reinterpret_cast<const float4*>(a.ws_u + row * P * DH) + d4;
  float mt = -INFINITY, lt = 0.0f;
  float4 ut = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = pg; p0 < P; p0 += 4 * NG) {
    float pm[4], pl[4];
    float4 pu[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int p = p0 + k * NG;
      const bool ok = p < P;
      pm[k] = ok ? ml[2 * p] : -INFINITY;
      pl[k] = ok ? ml[2 * p + 1] : 0.0f;
      pu[k] = ok ? u[(size_t)p * D4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mr = mt;
#pragma unroll
    for (int k = 0; k < 4; ++k) mr = fmaxf(mr, pm[k]);
    const float c = part_weight(mt, mr);
    lt *= c;
    ut.x *= c; ut.y *= c; ut.z *= c; ut.w *= c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float wgt = part_weight(pm[k], mr);
      lt = fmaf(wgt, pl[k], lt);
      if (wgt > 0.0f) {   // an empty partition's u is never read into the sum
        ut.x = fmaf(wgt, pu[k].x, ut.x); ut.y = fmaf(wgt, pu[k].y, ut.y);
        ut.z = fmaf(wgt, pu[k].z, ut.z); ut.w = fmaf(wgt, pu[k].w, ut.w);
      }
    }
    mt = mr;
  }
  s_u[pg][d4] = ut;
  if (d4 == 0) { s_m[pg] = mt; s_l[pg] = lt; }
  __syncthreads();
  if (t < D4) {
    float m = s_m[0];
#pragma unroll
    for (int q = 1; q < NG; ++q) m = fmaxf(m, s_m[q]);
    float l = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const float wgt = part_weight(s_m[q], m);
      l = fmaf(wgt, s_l[q], l);
      const float4 x = s_u[q][t];
      o.x = fmaf(wgt, x.x, o.x); o.y = fmaf(wgt, x.y, o.y); o.z = fmaf(wgt, x.z, o.z); o.w = fmaf(wgt, x.w, o.w);
    }
    const float4 r = l > 0.0f ? make_float4(o.x / l, o.y / l, o.z / l, o.w / l) : make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(a.out + row * DH)[t] = r;
  }
}

// ---- matrix-core form -------------------------------------------------------------
// The same (sequence, KV head, partition) work with the products on MFMA:
// the query heads of a KV group are the N dimension of 16×16 products, so a
// workgroup takes up to 16 heads of a group, and keys go 32 at a time (two
// blocks). For a pair of blocks:
//   Sᵀ = K·Qᵀ on v_mfma_f32_16x16x32_bf16, keys as M (16 per block), Dh as the
//   contraction: lane (col = lane % 16, kg = lane / 16) loads, for k-step dc,
//   8 elements of key row col (which 8 is MfmaGeometry::k_elem; the
//   contraction may take Dh in any order as long as q follows it); q of head
//   col is the B operand. K comes from memory in whole rows per load (CPR
//   lanes per row, so every request covers full cache lines) and is restaged
//   through a padded per-wave LDS area into that operand layout. The result
//   leaves in lane (col, kg) the scores of head col for keys 4kg … 4kg+3 of
//   each block.
//   Oᵀ += Vᵀ·Pᵀ on the same instruction with the 32 keys as the contraction:
//   those scores, as probabilities, are already the B operand (element j < 4
//   ↔ key 4kg+j of the first block, j ≥ 4 ↔ key 4kg+j−4 of the second). For
//   the A operand lane (col, kg) loads the NDT = Dh/16 consecutive elements
//   col·NDT … of its 4 keys of each block and transposes them in registers,
//   so output tile dt row m is column NDT·m + dt (a permutation of Dh that the
//   final store undoes). P enters as a bf16 high part (truncated) plus the
//   bf16 rounding of the remainder, two products, keeping ~16-bit
//   probabilities; K, V (fp8 converted exactly) and q are exact in bf16.
// The online softmax per head is the one above (log2 domain, lazy rescale,
// wave-uniform decision); the waves merge through LDS and write the output
// or the same partials for the reduce kernel.
// "Blocks" here are 16-row units: a pool block of 32 or 64 tokens holds two
// or four of them. The same kernel also runs (template flags) the decode
// step's append (APPEND: each sequence's new token is written to its slot
// and attended from the input), a mixed step's extra appends (EXTRA: the
// grid's last workgroups store prefill-chunk tokens) and the chunked prefill
// for small chunks (PREFILL: the 16 columns are (query head, query) pairs,
// each masked causally at its own position).
constexpr int kMfmaHeads = 16;   // query heads per workgroup (the MFMA N dimension)

template <int KV, int DH>
struct MfmaGeometry {
  static constexpr int ESZ = KV == kBF16 ? 2 : 1;   // stored bytes per element
  static constexpr int RB = DH * ESZ;               // bytes of one token row of one head
  static constexpr int NDC = DH / 32;               // k-steps of Sᵀ = K·Qᵀ
  static constexpr int NDT = DH / 16;               // 16-row tiles of Oᵀ = elements of a V slice
  static constexpr int KW = 8 * ESZ / 4;            // stored dwords of one K operand slice
  static constexpr int CPR = RB / 16;               // 16-byte chunks of a row
  static constexpr int RPI = kWave / CPR;           // rows per whole-row K load
  static constexpr int NKI = kBlockSize / RPI;      // whole-row K loads per block
  static constexpr int KRS = RB + 16;               // padded K row in LDS (bytes)
  static constexpr int VW = NDT * ESZ / 4;          // stored dwords of one V slice (≥ 1)
  static_assert(VW >= 1 && NDC >= 2, "unsupported head dimension");
  // First element of the 8 that lane group kg holds at k-step dc (the
  // contraction over Dh may take its elements in any order, as long as q and
  // K agree). Each K load covers 64 contiguous bytes of every row it touches:
  // bf16 — k-step dc, group kg holds chunk 4dc + kg of 16 bytes (8 elements);
  // fp8 — a 16-byte load of chunk 4·(dc/2) + kg holds 16 elements, the first
  // 8 for even dc and the last 8 for odd dc.
  static __device__ __forceinline__ int k_elem(int dc, int kg) {
    return KV == kFP8 ? (dc / 2) * 64 + kg * 16 + (dc % 2) * 8 : dc * 32 + kg * 8;
  }
};

// n stored dwords (n = 1, 2 or 4) at a byte offset, with cache policy AUX.
template <int N, int AUX = kCacheNonTemporal>
__device__ __forceinline__ void load_dwords(__amdgpu_buffer_rsrc_t r, int off, uint32_t (&d)[N]) {
  if constexpr (N == 4) {
    const uint4 x = buffer_load16_aux<AUX>(r, off);
    d[0] = x.x; d[1] = x.y; d[2] = x.z; d[3] = x.w;
  } else if constexpr (N == 2) {
    const uint2 x = buffer_load8_aux<AUX>(r, off);
    d[0] = x.x; d[1] = x.y;
  } else {
    d[0] = buffer_load4_aux<AUX>(r, off);
  }
}

// Stored dwords of a slice → packed bf16 pairs (fp8: two pairs per dword, exact).
template <int KV, int N>
__device__ __forceinline__ void to_bf16_pairs(const uint32_t (&x)[N], uint32_t (&y)[KV == kFP8 ? 2 * N : N]) {
  if constexpr (KV == kFP8) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      y[2 * i] = fp8x2_to_bf16x2<false>(x[i]);
      y[2 * i + 1] = fp8x2_to_bf16x2<true>(x[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = x[i];
  }
}

// n consecutive input elements (bf16 or fp32) from `base` as floats.
template <int N>
__device__ __forceinline__ void load_floats(const uint8_t* base, size_t elem, int dtype, float (&f)[N]) {
  if (dtype == kF32) {
    const float* p = reinterpret_cast<const float*>(base) + elem;
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + i);
      f[i] = x.x; f[i + 1] = x.y; f[i + 2] = x.z; f[i + 3] = x.w;
    }
  } else {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(base) + elem;
#pragma unroll
    for (int i = 0; i < N; i += 8) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + i);
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) { f[i + 2 * k] = bf16_lo(w[k]); f[i + 2 * k + 1] = bf16_hi(w[k]); }
    }
  }
}

// The stored bytes of n elements of the new token, starting at element
// `elem` of its row: a copy for bf16 caches (bf16 input), e4m3 of x·inv for
// fp8 caches — the same bits the append kernels store. N_BYTES is 4, 8 or 16.
template <int KV, int N_BYTES>
__device__ __forceinline__ void new_token_bytes(const uint8_t* base, size_t elem, int dtype, float inv,
                                                uint32_t (&out)[N_BYTES / 4]) {
  if constexpr (KV == kBF16) {
    const uint8_t* p = base + elem * 2;
    if constexpr (N_BYTES == 16) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      out[0] = x.x; out[1] = x.y;
    }
  } else {
    constexpr int N = N_BYTES;   // one byte per element
    float f[N < 8 ? 8 : N];
    if constexpr (N >= 8) {
      load_floats<N>(base, elem, dtype, f);
    } else {   // 4 elements
      if (dtype == kF32) {
        const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
        f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + elem);
        f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x); f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
      }
    }
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      uint32_t b = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) b |= encode_e4m3(f[4 * i + j] * inv) << (8 * j);
      out[i] = b;
    }
  }
}

// A mixed step's further appends: extra workgroup idx takes TOK tokens of
// one sequence (a.x_wgs_per_seq workgroups per sequence), NTH / TOK threads
// per token, each token stored exactly as the append kernels store it.
constexpr int kExtraTokens = 16;
template <int KV, int DH, int NTH, int TOK = kExtraTokens>
__device__ __forceinline__ void extra_append(const KernelArgs& a, int idx) {
  constexpr int per = NTH / TOK;
  const int s = idx / a.x_wgs_per_seq, j = idx % a.x_wgs_per_seq;
  if (s >= a.x_seqs) return;
  const int lo = a.x_cu[s], C = a.x_cu[s + 1] - lo;
  const int i = j * TOK + (int)threadIdx.x / per;
  if (i >= C) return;
  const int slot = slot_of(a.x_tables + (size_t)s * a.x_max_blocks, a.x_max_blocks, a.x_lens[s] - C + i,
                           a.block_size);
  const int t0 = (int)threadIdx.x % per;
  if constexpr (KV == kFP8) {
    if (a.new_dtype == kF32) {
      append_token<kF32, KV>(a.x_k, a.x_v, lo + i, slot, a.kc, a.vc, a.num_blocks, a.hkv, DH, a.k_inv, a.v_inv,
                             t0, per, a.block_size);
      return;
    }
  }
  append_token<kBF16, KV>(a.x_k, a.x_v, lo + i, slot, a.kc, a.vc, a.num_blocks, a.hkv, DH, a.k_inv, a.v_inv, t0,
                          per, a.block_size);
}

// Each wave's LDS region first stages its K blocks (two padded 16-row
// blocks), then, after its loop, holds its accumulators for the merge.
template <int KV, int DH>
constexpr int mfma_region_bytes() {
  using G = MfmaGeometry<KV, DH>;
  constexpr int kStage = 2 * kBlockSize * G::KRS;
  constexpr int kSlab = 4 * 4 * kMfmaHeads + 1;   // floats per dt slab of the accumulators (see the merge)
  return kStage > G::NDT * kSlab * 4 ? kStage : G::NDT * kSlab * 4;
}
// LDS of a workgroup of NW waves: the regions, then each wave's m and l per head
template <int KV, int DH, int NW>
constexpr int mfma_lds_bytes() { return NW * mfma_region_bytes<KV, DH>() + 2 * NW * kMfmaHeads * 4; }

// The matrix-core decode's work for workgroup `flat` of `nflat` (ids in the
// hardware's order), on NW waves and mfma_lds_bytes<KV, DH, NW>() bytes of
// LDS at `lds` (16-byte aligned).
template <int KV, int DH, int NW, bool APPEND, bool EXTRA, bool PREFILL = false, bool SPLIT8 = false>
__device__ __forceinline__ void decode_mfma_body(const KernelArgs& a, uint8_t* lds, uint32_t flat, uint32_t nflat) {
  constexpr int kWaves = NW, kThreads = NW * kWave;
  constexpr int NH = kMfmaHeads;
  using G = MfmaGeometry<KV, DH>;
  constexpr int NDC = G::NDC, NDT = G::NDT, KW = G::KW, VW = G::VW;
  constexpr int kSlab = 4 * 4 * NH + 1;        // floats per dt slab of the accumulators (see the merge)
  constexpr int kRegion = mfma_region_bytes<KV, DH>();
  auto sh_region = reinterpret_cast<uint8_t(*)[kRegion]>(lds);
  auto sh_m = reinterpret_cast<float(*)[NH]>(lds + kWaves * kRegion);
  auto sh_l = reinterpret_cast<float(*)[NH]>(lds + kWaves * kRegion + kWaves * NH * 4);

  if constexpr (EXTRA) {   // the last x_wgs workgroups only append; they fill the decode's ragged tail
    nflat -= a.x_wgs;
    if (flat >= nflat) {
      extra_append<KV, DH, kThreads>(a, (int)(flat - nflat));
      return;
    }
  }
  // prefill query blocks of one (sequence, KV head) share K/V: contiguous per XCD
  const uint32_t L = PREFILL ? xcd_logical_index(flat, nflat) : grouped_xcd_index(flat, nflat, decode_xcd_group(a));
  // decode: (sequence b, KV head g, head chunk, partition); prefill: (sequence
  // b, KV head g, head chunk, query block qb), one partition over all keys
  const int inner = PREFILL ? a.p_nqb : a.num_parts;
  const int chunk = (L / (PREFILL ? a.p_nqb : 1)) % a.num_chunks;
  const int part = PREFILL ? 0 : (L / a.num_chunks) % a.num_parts;
  const int qblk = PREFILL ? L % a.p_nqb : 0;
  const int g = (L / a.num_chunks / inner) % a.hkv;
  const int b = L / a.num_chunks / inner / a.hkv;
  const int group = a.hq / a.hkv;
  // prefill columns: head (col mod HG) of the chunk's HG heads, query qb·QB + col / HG
  const int hg_shift = PREFILL ? a.p_hg_shift : 0;
  const int h0 = PREFILL ? g * group + (chunk << hg_shift) : g * group + chunk * NH;
  const int nh = PREFILL ? NH : min(NH, group - chunk * NH);   // columns of this workgroup

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int col = lane & 15, kg = lane >> 4;
  const int P = a.num_parts;
  const int tok0 = part * a.part_tokens;
  // The kernel works in 16-row units ("blocks" below); a pool block of
  // bs = 16, 32 or 64 tokens holds bs/16 of them, unit u at rows
  // (u mod bs/16)·16 … of table entry u / (bs/16). With 8-token blocks
  // (SPLIT8) unit u is the 8 rows of entry 2u followed by the 8 rows of
  // entry 2u + 1: lanes 0-31 (key groups 0, 1) hold keys of the first, lanes
  // 32-63 keys of the second, and every load that would span both is issued
  // once per half-wave, each half with its own block's buffer resource.
  const int bs = a.block_size;
  const int unit_shift =
      SPLIT8 ? 0 : __builtin_amdgcn_readfirstlane(__builtin_ctz((unsigned)bs / kBlockSize));   // log2(bs/16)
  const int unit_mask = (1 << unit_shift) - 1;
  const size_t head_stride = (size_t)bs * G::RB;              // bytes of one (pool block, head)
  // Table entries, loaded beside the length: wave w takes unit pairs
  // (tiles) w, w + kWaves, …; lane j holds unit 2·(w + kWaves·(j/2)) + j%2.
  const int lb0 = tok0 / kBlockSize;                         // the partition's first unit
  const int units_in_table = SPLIT8 ? (a.max_blocks + 1) / 2 : a.max_blocks << unit_shift;
  const int cap = min(a.part_tokens / kBlockSize, units_in_table - lb0);
  const int jb = 2 * (w + kWaves * (lane >> 1)) + (lane & 1);
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks;
  const int phys_all = jb < cap ? bt[SPLIT8 ? 2 * (lb0 + jb) : (lb0 + jb) >> unit_shift] : -1;
  // SPLIT8: the unit's second block (entry 2u + 1, which may lie past the table)
  const int phys_all2 = SPLIT8 && jb < cap && 2 * (lb0 + jb) + 1 < a.max_blocks ? bt[2 * (lb0 + jb) + 1] : -1;
  auto unit_row0 = [&](int idx) { return SPLIT8 ? 0 : ((lb0 + idx) & unit_mask) * kBlockSize; };   // first pool row
  // the length through a vector-memory load: the scalar-cache wait for it
  // would also hold back every other scalar load issued before the first tile
  const int seq_len = (int)__builtin_amdgcn_raw_buffer_load_b32(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.seq_lens + b), 0, 4, kBufferRsrcWord3), 0, 0, 0);
  int q_lo = 0, n_q = 0;   // prefill: the sequence's first query row and its query count C
  if constexpr (PREFILL) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i qs = __builtin_amdgcn_raw_buffer_load_b64(
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.q_start + b), 0, 8, kBufferRsrcWord3), 0, 0, 0);
    q_lo = __builtin_amdgcn_readfirstlane(qs[0]);
    n_q = __builtin_amdgcn_readfirstlane(qs[1]) - q_lo;
  }
  constexpr int kAux = PREFILL ? 0 : kCacheNonTemporal;   // prefill items share K/V through L2


  auto tile_rsrc = [&](const uint8_t* pool, int phys, int row0, int rows) {
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const uint8_t* base = pool + ((size_t)(ok ? phys : 0) * a.hkv + g) * head_stride + (size_t)row0 * G::RB;
    const int records = __builtin_amdgcn_readfirstlane(ok ? rows * G::RB : 0);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, records, kBufferRsrcWord3);
  };
  struct Tile {
    uint4 k[2][G::NKI];       // [block][whole-row load]
    uint32_t v[2][4][VW];     // [block][key of the lane's quad]
  };
  // unit e of a tile: `rows` rows from row0 of table entry phys (SPLIT8: the
  // first 8 of them from entry phys, the rest from entry phys2)
  auto load_blocks = [&](Tile& t, int e, int phys, int phys2, int row0, int rows) {
    if constexpr (SPLIT8) {
      const auto rk0 = tile_rsrc(a.kc, phys, 0, min(rows, 8)), rk1 = tile_rsrc(a.kc, phys2, 0, max(rows - 8, 0));
      const auto rv0 = tile_rsrc(a.vc, phys, 0, min(rows, 8)), rv1 = tile_rsrc(a.vc, phys2, 0, max(rows - 8, 0));
      // K: a load of RPI ≤ 8 whole rows lies in one block; 16 rows (fp8, Dh=64) split by half-wave
#pragma unroll
      for (int i = 0; i < G::NKI; ++i) {
        const int row = i * G::RPI + lane / G::CPR, cb = (lane % G::CPR) * 16;
        if constexpr (G::RPI <= 8) {
          t.k[e][i] = buffer_load16_aux<kAux>(i * G::RPI < 8 ? rk0 : rk1, (row % 8) * G::RB + cb);
        } else {
          if (row < 8) t.k[e][i] = buffer_load16_aux<kAux>(rk0, row * G::RB + cb);
          else t.k[e][i] = buffer_load16_aux<kAux>(rk1, (row - 8) * G::RB + cb);
        }
      }
      // V: key group kg holds rows 4kg … 4kg+3, so lanes 0-31 read the first block, 32-63 the second
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (kg < 2) load_dwords<VW, kAux>(rv0, (4 * kg + i) * G::RB + col * VW * 4, t.v[e][i]);
        else load_dwords<VW, kAux>(rv1, (4 * kg - 8 + i) * G::RB + col * VW * 4, t.v[e][i]);
      }
    } else {
      const auto rk = tile_rsrc(a.kc, phys, row0, rows);
      const auto rv = tile_rsrc(a.vc, phys, row0, rows);
      // K: whole rows per load (CPR lanes per row), restaged through LDS
#pragma unroll
      for (int i = 0; i < G::NKI; ++i)
        t.k[e][i] = buffer_load16_aux<kAux>(rk, (i * G::RPI + lane / G::CPR) * G::RB + (lane % G::CPR) * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) load_dwords<VW, kAux>(rv, (4 * kg + i) * G::RB + col * VW * 4, t.v[e][i]);
    }
  };

  // The wave's first block pair is requested from its table entries alone,
  // all 16 rows of each, before the length arrives; the rows past the
  // sequence are masked when the pair is used.
  Tile first;
#pragma unroll
  for (int e = 0; e < 2; ++e)
    load_blocks(first, e, __builtin_amdgcn_readlane(phys_all, e), SPLIT8 ? __builtin_amdgcn_readlane(phys_all2, e) : -1,
                unit_row0(2 * w + e), kBlockSize);

  // q of column col as the B operand of each k-step (zeros for an unused column)
  const int qpb = NH >> hg_shift;                          // prefill: queries per query block
  const int my_qi = qblk * qpb + (col >> hg_shift);        // prefill: this lane's column's query
  bf16x8_t qb[NDC];
  if constexpr (PREFILL) {
    const bool ok = my_qi < n_q;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           ((size_t)(q_lo + (ok ? my_qi : 0)) * a.hq + h0 + (col & ((1 << hg_shift) - 1))) * DH;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      uint4 x = make_uint4(0, 0, 0, 0);
      if (ok) x = *reinterpret_cast<const uint4*>(qrow + G::k_elem(dc, kg));
      qb[dc] = __builtin_bit_cast(bf16x8_t, x);
    }
  } else {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.hq + h0 + (col < nh ? col : 0)) * DH;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + G::k_elem(dc, kg));
      qb[dc] = __builtin_bit_cast(bf16x8_t, col < nh ? x : make_uint4(0, 0, 0, 0));
    }
  }

  const int T = __builtin_amdgcn_readfirstlane(min(max(seq_len, 0), min(a.max_seq_len, a.max_blocks * bs)));
  // Keys the workgroup attends: decode, all T; prefill, up to its last
  // query's position (query i of the chunk sits at T − C + i, causal and
  // inclusive), each column masked at its own position.
  int kend = T, my_pos = 0;
  if constexpr (PREFILL) {
    const int qlast = min(n_q, (qblk + 1) * qpb) - 1;
    kend = __builtin_amdgcn_readfirstlane(qlast >= qblk * qpb ? max(0, T - n_q + qlast + 1) : 0);
    my_pos = T - n_q + my_qi;
  }
  const int ntok = min(a.part_tokens, kend - tok0);
  const int nblk = ntok > 0 ? (ntok + kBlockSize - 1) / kBlockSize : 0;
  const int ntile = (nblk + 1) / 2;
  const int ntw = ntile > w ? (ntile - w + kWaves - 1) / kWaves : 0;   // this wave's tiles
  const int my_phys = (lane >> 1) < ntw ? phys_all : -1;
  const int my_phys2 = SPLIT8 && (lane >> 1) < ntw ? phys_all2 : -1;
  float sc = a.scale_log2;
  if constexpr (KV == kFP8) sc *= a.k_scale[g];

  // Fused append: the sequence's new token sits at position T − 1. The
  // partition holding it reads that row from k_new / v_new (the stored bytes
  // the append writes) instead of the pool, and chunk 0's wave 0 writes it to
  // its slot; nothing in this launch reads the pool's copy of that row.
  int lb_new = -1, r_new = 0;
  uint4 knew = make_uint4(0, 0, 0, 0);   // lane (chunk lane % CPR) of the new K row, stored form
  uint32_t vnew[VW] = {};                // this lane's V slice (columns col·NDT …) of the new row
  if constexpr (APPEND) {
    const int pos = T - 1;
    if (pos >= tok0 && pos < tok0 + a.part_tokens) { lb_new = pos / kBlockSize - lb0; r_new = pos % kBlockSize; }
    if (T > 0) {
      const size_t row = ((size_t)b * a.hkv + g) * DH;   // element index of the new token's head-g row
      const float kinv = KV == kFP8 ? a.k_inv[g] : 1.0f, vinv = KV == kFP8 ? a.v_inv[g] : 1.0f;
      uint32_t kq[4];
      new_token_bytes<KV, 16>(a.k_new, row + (lane % G::CPR) * (16 / G::ESZ), a.new_dtype, kinv, kq);
      knew = make_uint4(kq[0], kq[1], kq[2], kq[3]);
      new_token_bytes<KV, VW * 4>(a.v_new, row + col * NDT, a.new_dtype, vinv, vnew);
    }
    if (lb_new >= 0 && chunk == 0 && w == 0) {
      const int phys = bt[pos / bs];
      if ((unsigned)phys < (unsigned)a.num_blocks) {
        const size_t off = ((size_t)phys * a.hkv + g) * head_stride + (size_t)(pos % bs) * G::RB;
        if (lane < G::CPR) *reinterpret_cast<uint4*>(a.kc + off + lane * 16) = knew;
        if (kg == 0) {
          uint8_t* vd = a.vc + off + col * VW * 4;
          if constexpr (VW == 4) *reinterpret_cast<uint4*>(vd) = make_uint4(vnew[0], vnew[1], vnew[2], vnew[3]);
          else if constexpr (VW == 2) *reinterpret_cast<uint2*>(vd) = make_uint2(vnew[0], vnew[1]);
          else *reinterpret_cast<uint32_t*>(vd) = vnew[0];
        }
      }
    }
  }

  auto rows_of = [&](int idx) { return min(kBlockSize, max(0, ntok - idx * kBlockSize)); };
  // block e (0, 1) of the wave's j-th tile
  auto block_phys = [&](int j, int e) { return j < ntw ? __builtin_amdgcn_readlane(my_phys, 2 * j + e) : -1; };
  auto block_phys2 = [&](int j, int e) {   // SPLIT8: the unit's second block
    return SPLIT8 && j < ntw ? __builtin_amdgcn_readlane(my_phys2, 2 * j + e) : -1;
  };
  auto block_index = [&](int j, int e) { return 2 * (w + kWaves * j) + e; };
  auto load_tile = [&](int j, Tile& t) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
      load_blocks(t, e, block_phys(j, e), block_phys2(j, e), unit_row0(block_index(j, e)), rows_of(block_index(j, e)));
  };

  float m_run = -INFINITY, l_run = 0.0f;     // head col; l is this lane's share
  f32x4_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto use_tile = [&](int j, const Tile& t) {
    // rmask[e] bit r: row r of unit e is a key to attend (inside the sequence,
    // in a block of the pool)
    uint32_t rmask[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = rows_of(block_index(j, e));
      if constexpr (SPLIT8) {
        const int r0 = (unsigned)block_phys(j, e) < (unsigned)a.num_blocks ? min(r, 8) : 0;
        const int r1 = (unsigned)block_phys2(j, e) < (unsigned)a.num_blocks ? max(r - 8, 0) : 0;
        rmask[e] = ((1u << r0) - 1u) | (((1u << r1) - 1u) << 8);
      } else {
        rmask[e] = (unsigned)block_phys(j, e) < (unsigned)a.num_blocks ? (1u << r) - 1u : 0u;
      }
    }
    // K rows to the wave's LDS stage, then back as the A operand (row col)
    uint8_t* stage = sh_region[w];
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < G::NKI; ++i)
        *reinterpret_cast<uint4*>(stage + (e * kBlockSize + i * G::RPI + lane / G::CPR) * G::KRS +
                                  (lane % G::CPR) * 16) = t.k[e][i];
    if constexpr (APPEND) {   // the new token's K row from k_new
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (block_index(j, e) == lb_new && lane < G::CPR)
          *reinterpret_cast<uint4*>(stage + (e * kBlockSize + r_new) * G::KRS + lane * 16) = knew;
    }
    wave_lds_sync();
    // Sᵀ for both blocks
    f32x4_t st[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint8_t* krow = stage + (e * kBlockSize + col) * G::KRS;
      uint32_t kd[NDC][KW];
      if constexpr (KV == kFP8) {   // a 16-byte piece holds two k-steps
#pragma unroll
        for (int d2 = 0; d2 < NDC / 2; ++d2) {
          const uint4 x = *reinterpret_cast<const uint4*>(krow + (d2 * 4 + kg) * 16);
          kd[2 * d2][0] = x.x; kd[2 * d2][1] = x.y;
          kd[2 * d2 + 1][0] = x.z; kd[2 * d2 + 1][1] = x.w;
        }
      } else {
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) {
          const uint4 x = *reinterpret_cast<const uint4*>(krow + (dc * 4 + kg) * 16);
          kd[dc][0] = x.x; kd[dc][1] = x.y; kd[dc][2] = x.z; kd[dc][3] = x.w;
        }
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        uint32_t kk[4];
        to_bf16_pairs<KV, KW>(kd[dc], kk);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(kk[0], kk[1], kk[2], kk[3])), qb[dc], acc, 0, 0, 0);
      }
      st[e] = acc;
    }
    // scale; keys past the valid rows (or of a block outside the pool) → −inf
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bool keep = (rmask[e] >> (4 * kg + i)) & 1u;
        if constexpr (PREFILL) keep = keep && block_index(j, e) * kBlockSize + 4 * kg + i <= my_pos;
        const float v = keep ? st[e][i] * sc : -INFINITY;
        st[e][i] = v;
        mt = fmaxf(mt, v);
      }
    mt = pair_halves32(pair_rows16(mt, MaxOp()), MaxOp());
    const float m_new = fmaxf(m_run, mt);
    if (__any(m_new > m_run)) {                          // rescale only when a max moved
      const float alpha = m_run == -INFINITY ? 0.0f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run == -INFINITY ? 0.0f : m_run;  // all keys so far masked: p = 0
    float pv[8];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pp = fast_exp2(st[e][i] - mc);
        pv[4 * e + i] = pp;
        l_run += pp;
      }
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u0 = __float_as_uint(pv[2 * i]), u1 = __float_as_uint(pv[2 * i + 1]);
      hw[i] = __builtin_amdgcn_perm(u1, u0, 0x07060302u);
      const float r0 = pv[2 * i] - __uint_as_float(u0 & 0xffff0000u);
      const float r1 = pv[2 * i + 1] - __uint_as_float(u1 & 0xffff0000u);
      lw[i] = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)r0, (__bf16)r1});
    }
    const bf16x8_t p_hi = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
    const bf16x8_t p_lo = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
    // V slices as bf16 pairs: vp[block][key][pair]
    constexpr int NP = NDT / 2;
    uint32_t vp[2][4][NP];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) to_bf16_pairs<KV, VW>(t.v[e][i], vp[e][i]);
    if (j == 0) {   // the first tile was read whole before the length was known: rows past it → 0
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q2 = 0; q2 < NP; ++q2) vp[e][i][q2] = (rmask[e] >> (4 * kg + i)) & 1u ? vp[e][i][q2] : 0u;
    }
    if constexpr (APPEND) {   // the new token's V slice from v_new
      uint32_t vn[NP];
      to_bf16_pairs<KV, VW>(vnew, vn);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        if (block_index(j, e) == lb_new)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q2 = 0; q2 < NP; ++q2) vp[e][i][q2] = 4 * kg + i == r_new ? vn[q2] : vp[e][i][q2];
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint32_t sel = dt % 2 ? 0x07060302u : 0x05040100u;   // high or low element of the pair
      uint32_t a4[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        a4[2 * e] = __builtin_amdgcn_perm(vp[e][1][dt / 2], vp[e][0][dt / 2], sel);
        a4[2 * e + 1] = __builtin_amdgcn_perm(vp[e][3][dt / 2], vp[e][2][dt / 2], sel);
      }
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, make_uint4(a4[0], a4[1], a4[2], a4[3]));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, p_hi, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, p_lo, o[dt], 0, 0, 0);
    }
  };

  {
    // The first pair is used on every path (a wave with no blocks sees it
    // fully masked, which adds nothing), so its loads stay ahead of the length.
    Tile t0 = first, t1;
    load_tile(1, t1);
    use_tile(0, t0);
    load_tile(2, t0);
    if (1 < ntw) use_tile(1, t1);
    for (int j = 2; j < ntw; j += 2) {
      load_tile(j + 1, t1);
      use_tile(j, t0);
      load_tile(j + 2, t0);
      if (j + 1 < ntw) use_tile(j + 1, t1);
    }
  }

  // ---- the wave's totals, then the waves' merge ------------------------------------
  l_run = pair_halves32(pair_rows16(l_run, AddOp()), AddOp());
  // The wave's accumulators go to its region as [dt][i][kg][head] with each dt
  // slab padded by one float: a store instruction (fixed dt, i) then covers 64
  // consecutive floats, and the merge's reads of consecutive columns d (dt
  // fastest) land in different banks.
  auto u_index = [](int dt, int i, int kgr, int h) { return dt * kSlab + (i * 4 + kgr) * NH + h; };
  wave_lds_sync();   // the wave's last stage reads are done before its region is reused
  float* my_u = reinterpret_cast<float*>(sh_region[w]);
  if (col < nh) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) my_u[u_index(dt, i, kg, col)] = o[dt][i];
    if (kg == 0) { sh_m[w][col] = m_run; sh_l[w][col] = l_run; }
  }
  __syncthreads();
  auto sh_u = [&](int ww, int h, int d) {   // column d = NDT·(4kg + i) + dt
    const int m = d / NDT;
    return reinterpret_cast<const float*>(sh_region[ww])[u_index(d % NDT, m % 4, m / 4, h)];
  };
  const float vscale = KV == kFP8 ? a.v_scale[g] : 1.0f;
  for (int i = tid; i < nh * DH; i += kThreads) {
    const int h = i / DH, d = i % DH;
    float mt = sh_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) mt = fmaxf(mt, sh_m[ww][h]);
    float u = 0.0f, lt = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float wt = part_weight(sh_m[ww][h], mt);
      u = fmaf(wt, sh_u(ww, h, d), u);
      lt = fmaf(wt, sh_l[ww][h], lt);
    }
    if constexpr (PREFILL) {
      const int qi = qblk * qpb + (h >> hg_shift);
      if (qi < n_q)
        a.out[((size_t)(q_lo + qi) * a.hq + h0 + (h & ((1 << hg_shift) - 1))) * DH + d] = lt > 0.0f ? u / lt : 0.0f;
    } else if (P == 1) {
      a.out[((size_t)b * a.hq + h0 + h) * DH + d] = lt > 0.0f ? u * vscale / lt : 0.0f;
    } else {
      a.ws_u[(((size_t)b * a.hq + h0 + h) * P + part) * DH + d] = u * vscale;
      if (d == 0) {
        float* ml = a.ws_ml + (((size_t)b * a.hq + h0 + h) * P + part) * 2;
        ml[0] = mt;
        ml[1] = lt;
      }
    }
  }
}


template <int KV, int DH, int NW, bool APPEND, bool EXTRA, bool PREFILL = false, bool SPLIT8 = false>
__global__ __launch_bounds__(NW * kWave) void decode_mfma_kernel(KernelArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[mfma_lds_bytes<KV, DH, NW>()];
  decode_mfma_body<KV, DH, NW, APPEND, EXTRA, PREFILL, SPLIT8>(a, lds, flat_block_id(), flat_grid_size());
}

// ---------------------------------------------------------------------------
// The mixed step in one launch ("06 KV Cache、Prefix Cache、PagedAttention 与
// vLLM", 6.6: one continuous-batching step mixes decodes and prefill chunks).
// Workgroups in the hardware's order: first the chunks' appends (kExtraTokens
// tokens each), then the decodes (each appending its own token), then the
// chunks' prefill query tiles. A prefill workgroup reads the chunk's keys
// from the pool, so it first waits until every append workgroup has
// published its stores: the appends count themselves into a slot of
// kMixedSlots counters (release at agent scope, which writes the XCD's L2
// back, once per workgroup), and the prefill's first lane polls the count,
// then acquires at agent scope (which invalidates stale lines) once. The hardware dispatches a grid's
// workgroups in order, so every append workgroup is resident or done before
// a prefill workgroup waits, and appends wait on nothing: the wait ends. It
// is bounded all the same (about a quarter second), so that a broken
// invariant costs a wrong result, not a hung GPU. The last prefill workgroup
// subtracts the counts back out, leaving the slot at zero for its next use.
constexpr int kMixedSlots = 1024;      // calls in flight per GPU, at most
constexpr int kMixedMaxSpins = 1 << 20;
__device__ unsigned mixed_sync[kMixedSlots][2];   // [slot]: appends done, prefill workgroups done

struct MixedLayout {
  uint32_t n_app, n_dec, n_dec_pad, n_pf, slot;
  uint32_t n_app_pad, n_pf_pad;   // the paired form: appends and prefill rounded up to the XCD rotation
};

// An append workgroup's stores are done: every wave's stores reach the XCD's
// L2; then one release at agent scope writes the L2 back (a fence per wave
// would write it back once per wave) and counts the workgroup.
__device__ __forceinline__ void mixed_append_done(unsigned* sync) {
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// A prefill workgroup waits for the n_app append workgroups (bounded).
__device__ __forceinline__ void mixed_wait_appends(unsigned* sync, uint32_t n_app) {
  if (threadIdx.x == 0) {
    for (int spins = 0; spins < kMixedMaxSpins; ++spins) {
      if (__hip_atomic_load(&sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_app) break;
      __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // one invalidate, not one per poll
  }
  __syncthreads();
}

// The paired form's prefill waves wait for the appends only before their
// first request of a tile that holds chunk keys (the prefix before it is in
// the pool already): each wave polls, then acquires at agent scope.
struct AppendGate {
  static constexpr bool kActive = true;
  unsigned* sync;
  uint32_t n_app;
  __device__ void wait() const {
    for (int spins = 0; spins < kMixedMaxSpins; ++spins) {
      if (__hip_atomic_load(&sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= n_app) break;
      __builtin_amdgcn_s_sleep(8);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
};

// A prefill workgroup is done; the last of n_pf returns the slot to zero.
__device__ __forceinline__ void mixed_prefill_done(unsigned* sync, uint32_t n_app, uint32_t n_pf) {
  __syncthreads();
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(&sync[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == n_pf - 1) {
    __hip_atomic_fetch_sub(&sync[0], n_app, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_sub(&sync[1], n_pf, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int DH>
constexpr int mixed_lds_bytes() {
  constexpr int d = mfma_lds_bytes<kBF16, DH, kDecodeWaves>(), p = stream_lds_bytes<DH, kStreams>();
  return d > p ? d : p;
}

template <int DH>
__global__ __launch_bounds__(kDecodeWaves * kWave, 1) void mixed_step_kernel(KernelArgs a, SArgs pa, MixedLayout m) {
  static_assert(kDecodeWaves == 2 * kStreams, "one workgroup size for both bodies");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[mixed_lds_bytes<DH>()];
  unsigned* sync = mixed_sync[m.slot];
  const uint32_t flat = flat_block_id();
  if (flat < m.n_app) {
    extra_append<kBF16, DH, kDecodeWaves * kWave>(a, (int)flat);
    mixed_append_done(sync);
    return;
  }
  if (flat < m.n_app + m.n_dec_pad) {
    const uint32_t id = flat - m.n_app;
    if (id < m.n_dec) decode_mfma_body<kBF16, DH, kDecodeWaves, true, false>(a, lds, id, m.n_dec);
    return;
  }
  mixed_wait_appends(sync, m.n_app);
  prefill_stream_body<DH, kStreams>(pa, lds, xcd_logical_index(flat - m.n_app - m.n_dec_pad, m.n_pf));
  mixed_prefill_done(sync, m.n_app, m.n_pf);
}

// The paired form: four-wave workgroups small enough (registers, at most
// 80 KiB of LDS) for two to share a CU, ordered appends, then the prefill
// query tiles (two key streams of two row groups, rings of three K and two
// V slots), then the decodes. The first round of dispatch gives each CU a
// prefill tile, the second a decode unit beside it, so the matrix-core
// prefill and the memory-bound decode overlap on every CU. The decodes'
// workgroups take at most 64·16·4 tokens each (their table covers 64 units
// per wave).
constexpr int kPairWaves = 4;
constexpr int kPairPrefillKmax = 3;
constexpr int kPairExtraTokens = 16;   // tokens per append workgroup (4 measured slower: more L2 write-backs)
constexpr int kPairMaxPartition = 64 * kBlockSize * kPairWaves;

template <int DH>
constexpr int mixed_pair_lds_bytes() {
  constexpr int d = mfma_lds_bytes<kBF16, DH, kPairWaves>(), p = stream_lds_bytes<DH, 2, 2, kPairPrefillKmax>();
  return d > p ? d : p;
}

template <int DH>
__global__ __launch_bounds__(kPairWaves * kWave, 2) void mixed_pair_kernel(KernelArgs a, SArgs pa, MixedLayout m) {
  static_assert(2 * mixed_pair_lds_bytes<DH>() <= 160 * 1024, "two workgroups per CU");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[mixed_pair_lds_bytes<DH>()];
  unsigned* sync = mixed_sync[m.slot];
  const uint32_t flat = flat_block_id();
  if (flat < m.n_app_pad) {
    if (flat < m.n_app) {
      extra_append<kBF16, DH, kPairWaves * kWave, kPairExtraTokens>(a, (int)flat);
      mixed_append_done(sync);
    }
    return;
  }
  if (flat >= m.n_app_pad + m.n_pf_pad) {
    const uint32_t id = flat - m.n_app_pad - m.n_pf_pad;
    if (id < m.n_dec) decode_mfma_body<kBF16, DH, kPairWaves, true, false>(a, lds, id, m.n_dec);
    return;
  }
  const uint32_t pid = flat - m.n_app_pad;
  if (pid >= m.n_pf) return;
  prefill_stream_body<DH, 2, 2, false, kPairPrefillKmax>(pa, lds, xcd_logical_index(pid, m.n_pf),
                                                         AppendGate{sync, m.n_app});
  mixed_prefill_done(sync, m.n_app, m.n_pf);
}

// The one launch for small chunks, whose prefill takes the column form (the
// decode body with (query head, query) columns): appends, decodes, then the
// chunks' query blocks, all eight-wave workgroups of the same body, so the
// query blocks fill the decodes' ragged tail. The query blocks wait for the
// appends as the eight-wave form's prefill does (they are last in the grid:
// the appends are done by then). Bit-identical to the separate calls.
template <int DH>
__global__ __launch_bounds__(kDecodeWaves * kWave) void mixed_cols_kernel(KernelArgs a, KernelArgs ca,
                                                                          MixedLayout m) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[mfma_lds_bytes<kBF16, DH, kDecodeWaves>()];
  unsigned* sync = mixed_sync[m.slot];
  const uint32_t flat = flat_block_id();
  if (flat < m.n_app) {
    extra_append<kBF16, DH, kDecodeWaves * kWave>(a, (int)flat);
    mixed_append_done(sync);
    return;
  }
  if (flat < m.n_app + m.n_dec_pad) {
    const uint32_t id = flat - m.n_app;
    if (id < m.n_dec) decode_mfma_body<kBF16, DH, kDecodeWaves, true, false>(a, lds, id, m.n_dec);
    return;
  }
  mixed_wait_appends(sync, m.n_app);
  decode_mfma_body<kBF16, DH, kDecodeWaves, false, false, true>(ca, lds, flat - m.n_app - m.n_dec_pad, m.n_pf);
  mixed_prefill_done(sync, m.n_app, m.n_pf);
}

// Lanes per K row: 4 keeps the score reduction to two DPP steps and one
// exponential per lane and head; eight heads per workgroup take 8 so that
// their q slices fit in fewer registers.
template <int HC>
constexpr int k_lanes() { return HC >= 8 ? 8 : 4; }

template <int KV, int DH, int HC>
hipError_t launch_t(const DecodeParams& p, const KernelArgs& a, hipStream_t s) {
  const size_t n = (size_t)p.batch * p.cache.num_kv_heads * a.num_chunks * p.num_parts;
  hipLaunchKernelGGL((decode_split_kernel<KV, DH, HC, k_lanes<HC>(), kDecodeWaves>), dim3((unsigned)n),
                     dim3(kDecodeWaves * kWave), 0, s, a);
  return hipGetLastError();
}

template <int KV, int DH>
hipError_t launch_mfma(const DecodeParams& p, const KernelArgs& a, hipStream_t s) {
  const size_t n = (size_t)p.batch * p.cache.num_kv_heads * a.num_chunks * p.num_parts;
  const dim3 block(kDecodeWaves * kWave);
  if (a.x_wgs > 0) {
    if constexpr (KV == kBF16) {
      if (a.block_size == 8)
        hipLaunchKernelGGL((decode_mfma_kernel<KV, DH, kDecodeWaves, true, true, false, true>),
                           dim3((unsigned)(n + a.x_wgs)), block, 0, s, a);
      else
        hipLaunchKernelGGL((decode_mfma_kernel<KV, DH, kDecodeWaves, true, true>), dim3((unsigned)(n + a.x_wgs)),
                           block, 0, s, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;   // the mixed step takes bf16 caches only
  }
  if (a.block_size == 8) {   // 16-row units over pairs of 8-token blocks
    if (a.k_new)
      hipLaunchKernelGGL((decode_mfma_kernel<KV, DH, kDecodeWaves, true, false, false, true>), dim3((unsigned)n), block,
                         0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<KV, DH, kDecodeWaves, false, false, false, true>), dim3((unsigned)n),
                         block, 0, s, a);
    return hipGetLastError();
  }
  if (a.k_new)
    hipLaunchKernelGGL((decode_mfma_kernel<KV, DH, kDecodeWaves, true, false>), dim3((unsigned)n), block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<KV, DH, kDecodeWaves, false, false>), dim3((unsigned)n), block, 0, s, a);
  return hipGetLastError();
}

template <int KV, int DH>
hipError_t launch_hc(const DecodeParams& p, const KernelArgs& a, int hc, hipStream_t s) {
  switch (hc) {
    case 1: return launch_t<KV, DH, 1>(p, a, s);
    case 2: return launch_t<KV, DH, 2>(p, a, s);
    case 4: return launch_t<KV, DH, 4>(p, a, s);
    default: return launch_t<KV, DH, 8>(p, a, s);
  }
}

}  // namespace

int decode_heads_per_wg(int group, int kernel) {
  if (kernel == kDecodeMatrix) return kMfmaHeads;
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

namespace {

// The column form's arguments (the prefill on the decode body); *n: its
// workgroups. False when the call does not fit the form.
bool make_cols_args(const PrefillParams& p, KernelArgs* out, size_t* n) {
  const int hkv = p.cache.num_kv_heads, group = p.num_q_heads / hkv;
  const int hg = prefill_cols_heads(group);
  const int64_t keys = (int64_t)p.max_blocks * p.cache.block_size;
  if (keys > kPrefillColsMaxKeys || p.cache.block_size < kBlockSize || p.cache.dtype != kBF16) return false;
  KernelArgs a = {};
  a.kc = static_cast<uint8_t*>(p.cache.k);
  a.vc = static_cast<uint8_t*>(p.cache.v);
  a.q = p.q;
  a.block_tables = p.block_tables;
  a.seq_lens = p.seq_lens;
  a.out = p.out;
  a.num_blocks = p.cache.num_blocks;
  a.hkv = hkv;
  a.hq = p.num_q_heads;
  a.max_blocks = p.max_blocks;
  a.max_seq_len = (int)keys;
  a.part_tokens = (int)keys;
  a.num_parts = 1;
  a.num_chunks = group / hg;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.block_size = p.cache.block_size;
  a.q_start = p.q_start;
  a.p_hg_shift = __builtin_ctz((unsigned)hg);
  a.p_nqb = (p.max_q_len + kMfmaHeads / hg - 1) / (kMfmaHeads / hg);
  *out = a;
  *n = (size_t)p.num_seqs * hkv * a.num_chunks * a.p_nqb;
  return true;
}

KernelArgs make_kernel_args(const DecodeParams& p) {
  const int group = p.num_q_heads / p.cache.num_kv_heads;
  const int hc = decode_heads_per_wg(group, p.kernel);
  KernelArgs a{};
  a.kc = static_cast<uint8_t*>(p.cache.k);
  a.vc = static_cast<uint8_t*>(p.cache.v);
  a.k_scale = p.cache.k_scale;
  a.v_scale = p.cache.v_scale;
  a.q = p.q;
  a.block_tables = p.block_tables;
  a.seq_lens = p.seq_lens;
  a.out = p.out;
  a.ws_ml = p.ws_ml;
  a.ws_u = p.ws_u;
  a.num_blocks = p.cache.num_blocks;
  a.hkv = p.cache.num_kv_heads;
  a.hq = p.num_q_heads;
  a.max_blocks = p.max_blocks;
  a.max_seq_len = p.max_seq_len;
  a.part_tokens = p.part_tokens;
  a.num_parts = p.num_parts;
  a.num_chunks = (group + hc - 1) / hc;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.k_new = p.kernel == kDecodeMatrix ? static_cast<const uint8_t*>(p.k_new) : nullptr;
  a.v_new = static_cast<const uint8_t*>(p.v_new);
  a.k_inv = p.k_inv;
  a.v_inv = p.v_inv;
  a.new_dtype = p.new_dtype;
  a.block_size = p.cache.block_size;
  a.x_k = static_cast<const uint8_t*>(p.x_k);
  a.x_v = static_cast<const uint8_t*>(p.x_v);
  a.x_cu = p.x_cu;
  a.x_lens = p.x_lens;
  a.x_tables = p.x_tables;
  a.x_max_blocks = p.x_max_blocks;
  a.x_seqs = p.x_seqs;
  a.x_wgs_per_seq = (p.x_max_q + kExtraTokens - 1) / kExtraTokens;
  a.x_wgs = p.x_seqs > 0 && a.x_wgs_per_seq > 0 ? (p.x_seqs * a.x_wgs_per_seq + 7) / 8 * 8 : 0;
  return a;
}

hipError_t launch_merge(const DecodeParams& p, hipStream_t s) {
  MergeArgs m;
  m.ws_ml = p.ws_ml;
  m.ws_u = p.ws_u;
  m.out = p.out;
  m.num_parts = p.num_parts;
  const unsigned rows = (unsigned)((size_t)p.batch * p.num_q_heads);
  if (p.cache.head_dim == 64) hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(rows), dim3(kMergeThreads), 0, s, m);
  else hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(rows), dim3(kMergeThreads), 0, s, m);
  return hipGetLastError();
}

std::atomic<uint32_t> g_mixed_slot{0};

template <int DH>
hipError_t launch_mixed_dh(const DecodeParams& dp, const PrefillParams& pp, bool pair, hipStream_t s) {
  KernelArgs a = make_kernel_args(dp);
  if (pair) {   // kPairExtraTokens tokens per append workgroup
    a.x_wgs_per_seq = (dp.x_max_q + kPairExtraTokens - 1) / kPairExtraTokens;
    a.x_wgs = dp.x_seqs > 0 && a.x_wgs_per_seq > 0 ? (dp.x_seqs * a.x_wgs_per_seq + 7) / 8 * 8 : 0;
  }
  const SArgs pa = make_sargs(pp);
  MixedLayout m;
  m.n_app = (uint32_t)a.x_wgs;
  m.n_dec = dp.batch > 0 ? (uint32_t)((size_t)dp.batch * dp.cache.num_kv_heads * a.num_chunks * dp.num_parts) : 0u;
  m.n_dec_pad = (m.n_dec + 7) / 8 * 8;      // keeps the prefill's ids aligned to the XCD rotation
  m.n_pf = (uint32_t)stream_workgroups(pp, pa);
  m.slot = g_mixed_slot.fetch_add(1, std::memory_order_relaxed) % kMixedSlots;
  m.n_app_pad = (m.n_app + 7) / 8 * 8;
  m.n_pf_pad = (m.n_pf + 7) / 8 * 8;
  hipError_t e;
  if (pair) {
    const size_t n = (size_t)m.n_app_pad + m.n_pf_pad + m.n_dec;
    if (n > (size_t)INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mixed_pair_kernel<DH>, dim3((unsigned)n), dim3(kPairWaves * kWave), 0, s, a, pa, m);
  } else {
    const size_t n = (size_t)m.n_app + m.n_dec_pad + m.n_pf;
    hipLaunchKernelGGL(mixed_step_kernel<DH>, dim3((unsigned)n), dim3(kDecodeWaves * kWave), 0, s, a, pa, m);
  }
  e = hipGetLastError();
  if (e != hipSuccess || dp.batch == 0 || dp.num_parts <= 1) return e;
  return launch_merge(dp, s);
}

}  // namespace

hipError_t launch_mixed_one(const DecodeParams& dp, const PrefillParams& pp, bool pair, hipStream_t s) {
  if (dp.kernel != kDecodeMatrix || dp.cache.dtype != kBF16 || pp.num_seqs == 0 || pp.max_q_len == 0)
    return hipErrorInvalidValue;
  if (pair && dp.batch > 0 && dp.part_tokens > kPairMaxPartition) return hipErrorInvalidValue;
  return dp.cache.head_dim == 64 ? launch_mixed_dh<64>(dp, pp, pair, s) : launch_mixed_dh<128>(dp, pp, pair, s);
}

size_t prefill_cols_workgroups(const PrefillParams& p) {
  KernelArgs a;
  size_t n = 0;
  return make_cols_args(p, &a, &n) ? n : 0;
}

hipError_t launch_mixed_cols(const DecodeParams& dp, const PrefillParams& pp, hipStream_t s) {
  if (dp.kernel != kDecodeMatrix || dp.cache.dtype != kBF16 || pp.num_seqs == 0 || pp.max_q_len == 0)
    return hipErrorInvalidValue;
  KernelArgs ca;
  size_t n_pf = 0;
  if (!make_cols_args(pp, &ca, &n_pf)) return hipErrorInvalidValue;
  const KernelArgs a = make_kernel_args(dp);
  MixedLayout m{};
  m.n_app = (uint32_t)a.x_wgs;
  m.n_dec = dp.batch > 0 ? (uint32_t)((size_t)dp.batch * dp.cache.num_kv_heads * a.num_chunks * dp.num_parts) : 0u;
  m.n_dec_pad = (m.n_dec + 7) / 8 * 8;      // keeps the query blocks' ids aligned to the XCD rotation
  m.n_pf = (uint32_t)n_pf;
  m.slot = g_mixed_slot.fetch_add(1, std::memory_order_relaxed) % kMixedSlots;
  const size_t n = (size_t)m.n_app + m.n_dec_pad + m.n_pf;
  if (n > (size_t)INT32_MAX) return hipErrorInvalidValue;
  const dim3 block(kDecodeWaves * kWave);
  if (dp.cache.head_dim == 64)
    hipLaunchKernelGGL(mixed_cols_kernel<64>, dim3((unsigned)n), block, 0, s, a, ca, m);
  else
    hipLaunchKernelGGL(mixed_cols_kernel<128>, dim3((unsigned)n), block, 0, s, a, ca, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || dp.batch == 0 || dp.num_parts <= 1) return e;
  return launch_merge(dp, s);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.batch == 0 && p.x_seqs == 0) return hipSuccess;
  const int group = p.num_q_heads / p.cache.num_kv_heads;
  const int hc = decode_heads_per_wg(group, p.kernel);
  const KernelArgs a = make_kernel_args(p);
  if (a.x_wgs > 0 && p.kernel != kDecodeMatrix) return hipErrorInvalidValue;
  const int dt = p.cache.dtype, dh = p.cache.head_dim;
  hipError_t e;
  if (p.kernel == kDecodeMatrix)
    e = dt == kBF16 ? (dh == 64 ? launch_mfma<kBF16, 64>(p, a, s) : launch_mfma<kBF16, 128>(p, a, s))
                    : (dh == 64 ? launch_mfma<kFP8, 64>(p, a, s) : launch_mfma<kFP8, 128>(p, a, s));
  else if (dt == kF32) e = dh == 64 ? launch_hc<kF32, 64>(p, a, hc, s) : launch_hc<kF32, 128>(p, a, hc, s);
  else if (dt == kBF16) e = dh == 64 ? launch_hc<kBF16, 64>(p, a, hc, s) : launch_hc<kBF16, 128>(p, a, hc, s);
  else e = dh == 64 ? launch_hc<kFP8, 64>(p, a, hc, s) : launch_hc<kFP8, 128>(p, a, hc, s);
  if (e != hipSuccess || p.batch == 0 || p.num_parts <= 1) return e;
  return launch_merge(p, s);
}

int prefill_cols_heads(int group) {
  int hg = 1;
  while (hg < kMfmaHeads && group % (2 * hg) == 0) hg *= 2;
  return hg;
}

// Split-KV scratch of pkv_attn_decode_noalloc, for callers that cannot
// allocate device memory. Each GPU that runs the library holds its own copy of
// this array until the process ends. Host code never passes `scratch` itself
// to a kernel (on the host the name stands for a host-side shadow, not a
// device address): the device address comes from hipGetSymbolAddress, looked
// up once per device with that device current and kept per device.
static __device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

hipError_t decode_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

hipError_t launch_prefill_cols(const PrefillParams& p, hipStream_t s) {
  if (p.num_seqs == 0 || p.max_q_len == 0) return hipSuccess;
  KernelArgs a;
  size_t n = 0;
  if (!make_cols_args(p, &a, &n)) return hipErrorInvalidValue;
  const dim3 block(kDecodeWaves * kWave);
  if (p.cache.head_dim == 64)
    hipLaunchKernelGGL((decode_mfma_kernel<kBF16, 64, kDecodeWaves, false, false, true>), dim3((unsigned)n), block, 0,
                       s, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<kBF16, 128, kDecodeWaves, false, false, true>), dim3((unsigned)n), block,
                       0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
