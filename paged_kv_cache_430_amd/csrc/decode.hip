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
// One workgroup (4 waves) owns (sequence b, KV head g, a chunk of HC query
// heads of that group, partition π of part_tokens tokens). Each wave streams
// the blocks w, w+4, w+8, … of π in a single pass:
//   * the wave's block-table entries are loaded once, one per lane, and read
//     back with a lane read into a scalar register;
//   * K and V of the next block are loaded while the current one is used
//     (16-byte loads; a token row of one head is read by row_bytes/16
//     consecutive lanes, so every load instruction covers whole rows);
//   * a lane holds an EPC-element column slice of several token rows; the
//     score of a (token, head) is the sum over the row's lanes (DPP), so every
//     lane of the row ends with it and multiplies its own V slice by p;
//   * online softmax per head in the log2 domain: the running max moves only
//     when a block raises it, and only then are l and the accumulators
//     rescaled (the wave-uniform branch is rarely taken once the max settles).
// At the end the wave's accumulators are summed over its row groups, the four
// waves are merged through LDS, and either o = u / l is written (one
// partition) or (m, l, u) go to the workspace for a second, small kernel that
// merges the partitions. (Merging in the last workgroup to finish would need
// a device-scope release per workgroup, which writes back the L2 of its XCD
// every time; the kernel boundary does that once.)
// Masked slots (past the sequence end) are selected out, never multiplied by
// zero, and blocks whose id is outside the pool are skipped: pool slots may
// hold NaN.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int KV, int DH>
struct Geometry {
  static constexpr int ESZ = KV == kF32 ? 4 : KV == kBF16 ? 2 : 1;  // stored bytes per element
  static constexpr int RB = DH * ESZ;         // bytes of one token row of one head
  static constexpr int LPR = RB / 16;         // lanes per row (16 bytes each)
  static constexpr int RPI = kWave / LPR;     // rows covered by one wave load
  static constexpr int NI = kBlockSize / RPI; // loads per block (per K or V)
  static constexpr int EPC = 16 / ESZ;        // elements in a lane's 16-byte slice
  // q dwords per head and lane: fp32 values, or packed bf16 pairs
  static constexpr int QD = KV == kF32 ? EPC : EPC / 2;
  static_assert(LPR >= 4 && LPR <= 32 && NI >= 1, "unsupported row size");
};

struct KernelArgs {
  const uint8_t* kc;
  const uint8_t* vc;
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
};

struct MergeArgs {
  const float* ws_ml;
  const float* ws_u;
  const int32_t* seq_lens;
  float* out;
  size_t total;   // batch · Hq · head_dim
  int hq, head_dim, max_blocks, max_seq_len, part_tokens, num_parts;
};

// Sum over the LPR consecutive lanes of a row (LPR = 4, 8, 16 or 32); every
// lane of the row receives the same bits (each step adds a commutative pair).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp_f32<kQuadXor1>(x);
  x += dpp_f32<kQuadXor2>(x);
  if constexpr (LPR >= 8) x += dpp_f32<kRowHalfMirror>(x);
  if constexpr (LPR >= 16) x += dpp_f32<kRowMirror>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16, kWave);
  return x;
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

// exp2 with exp2(−inf − x) taken as 0 also when x is −inf (an empty part).
__device__ __forceinline__ float part_weight(float m, float mt) {
  return m == -INFINITY ? 0.0f : fast_exp2(m - mt);
}

template <int KV, int DH, int HC>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(KernelArgs a) {
  using G = Geometry<KV, DH>;
  constexpr int NI = G::NI, EPC = G::EPC, QD = G::QD, LPR = G::LPR, RPI = G::RPI;
  __shared__ float sh_u[kWaves][HC][DH];
  __shared__ float sh_m[kWaves][HC];
  __shared__ float sh_l[kWaves][HC];

  // ---- which (b, g, chunk, partition) ----------------------------------------
  const uint32_t L = xcd_logical_index(flat_block_id(), flat_grid_size());
  const int chunk = L % a.num_chunks;
  const int part = (L / a.num_chunks) % a.num_parts;
  const int g = (L / a.num_chunks / a.num_parts) % a.hkv;
  const int b = L / a.num_chunks / a.num_parts / a.hkv;
  const int group = a.hq / a.hkv;
  const int h0 = g * group + chunk * HC;

  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int T = min(max(a.seq_lens[b], 0), min(a.max_seq_len, a.max_blocks * kBlockSize));
  const int nparts = (T + a.part_tokens - 1) / a.part_tokens;
  if (part >= nparts) {
    if (part == 0) {  // empty sequence: zeros
      for (int i = tid; i < HC * DH; i += kThreads) a.out[((size_t)b * a.hq + h0) * DH + i] = 0.0f;
    }
    return;
  }
  const int tok0 = part * a.part_tokens;
  const int ntok = min(a.part_tokens, T - tok0);
  const int nblk = (ntok + kBlockSize - 1) / kBlockSize;
  const int nbw = nblk > w ? (nblk - w + kWaves - 1) / kWaves : 0;   // this wave's blocks
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + tok0 / kBlockSize;
  const int my_phys = lane < nbw ? bt[w + kWaves * lane] : -1;
  const size_t head_stride = (size_t)kBlockSize * G::RB;     // bytes of one (block, head)

  const int r = lane / LPR, cc = lane % LPR;                  // row group, 16-byte column
  const int lane_off = r * G::RB + cc * 16;                  // within a (block, head) tile

  // q slices of the HC heads
  uint32_t qreg[HC][QD];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    const size_t row = (size_t)b * a.hq + h0 + h;
    if constexpr (KV == kF32) {
      const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.q) + row * DH + cc * EPC);
      qreg[h][0] = x.x; qreg[h][1] = x.y; qreg[h][2] = x.z; qreg[h][3] = x.w;
    } else {
      const uint16_t* qp = static_cast<const uint16_t*>(a.q) + row * DH + cc * EPC;
#pragma unroll
      for (int c = 0; c < QD / 4; ++c) {
        const uint4 x = *reinterpret_cast<const uint4*>(qp + 8 * c);
        qreg[h][4 * c] = x.x; qreg[h][4 * c + 1] = x.y; qreg[h][4 * c + 2] = x.z; qreg[h][4 * c + 3] = x.w;
      }
    }
  }
  float sc = a.scale_log2;
  if constexpr (KV == kFP8) sc *= a.k_scale[g];

  float m[HC], l[HC], acc[HC][EPC];
#pragma unroll
  for (int h = 0; h < HC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[h][e] = 0.0f;
  }

  // Buffer resources over the wave's j-th (block, head) tile of K and V. An id
  // outside the pool, and j past the wave's last block, give zero records:
  // their loads return zeros without touching memory, so loads need no branch.
  auto tile_rsrc = [&](const uint8_t* pool, int phys) {
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const uint8_t* base = pool + ((size_t)(ok ? phys : 0) * a.hkv + g) * head_stride;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, ok ? (int)head_stride : 0,
                                             kBufferRsrcWord3);
  };
  auto load_block = [&](int j, uint4 (&kb)[NI], uint4 (&vb)[NI]) {
    const int phys = __builtin_amdgcn_readlane(my_phys, j);
    const auto rk = tile_rsrc(a.kc, phys);
    const auto rv = tile_rsrc(a.vc, phys);
#pragma unroll
    for (int i = 0; i < NI; ++i) kb[i] = buffer_load16(rk, lane_off + i * RPI * G::RB);
#pragma unroll
    for (int i = 0; i < NI; ++i) vb[i] = buffer_load16(rv, lane_off + i * RPI * G::RB);
  };

  auto use_block = [&](int j, const uint4 (&kb)[NI], const uint4 (&vb)[NI]) {
    const int phys = __builtin_amdgcn_readlane(my_phys, j);
    if ((unsigned)phys >= (unsigned)a.num_blocks) return;     // contributes nothing
    const int lb = w + kWaves * j;                             // block within the partition
    const int valid_rows = ntok - lb * kBlockSize;             // >= 1
    // scores of the lane's NI tokens for the HC heads
    float s[HC][NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      uint32_t kk[QD];
      k_operand<KV, QD>(kb[i], kk);
#pragma unroll
      for (int h = 0; h < HC; ++h) s[h][i] = row_sum<LPR>(slice_dot<KV, QD>(qreg[h], kk, 0.0f)) * sc;
    }
    bool row_ok[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) row_ok[i] = r + RPI * i < valid_rows;
    if (valid_rows < kBlockSize) {                             // tail block: select out
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < HC; ++h) s[h][i] = row_ok[i] ? s[h][i] : -INFINITY;
    }
    // block max per head; rescale only when it raises the running max
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      float bm = s[h][0];
#pragma unroll
      for (int i = 1; i < NI; ++i) bm = fmaxf(bm, s[h][i]);
#pragma unroll
      for (int off = LPR; off < kWave; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off, kWave));
      if (bm > m[h]) {
        const float alpha = m[h] == -INFINITY ? 0.0f : fast_exp2(m[h] - bm);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] *= alpha;
        m[h] = bm;
      }
    }
    // p = 2^(s − m); l += p; acc += p · v (rows past the end are zero-filled
    // by the tile's record limit only for whole blocks, so select them out)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float f[EPC];
      slice_values<KV, EPC>(vb[i], f);
      if (valid_rows < kBlockSize) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) f[e] = row_ok[i] ? f[e] : 0.0f;
      }
#pragma unroll
      for (int h = 0; h < HC; ++h) {
        const float p = fast_exp2(s[h][i] - m[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[h][e] = fmaf(p, f[e], acc[h][e]);
      }
    }
  };

  {
    uint4 k0[NI], v0[NI], k1[NI], v1[NI];
    load_block(0, k0, v0);
    for (int j = 0; j < nbw; j += 2) {
      load_block(j + 1, k1, v1);
      use_block(j, k0, v0);
      load_block(j + 2, k0, v0);
      if (j + 1 < nbw) use_block(j + 1, k1, v1);
    }
  }

  // ---- the wave's totals: sum over its row groups ----------------------------
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      l[h] += __shfl_xor(l[h], off, kWave);
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, kWave);
    }
  }
  // every lane of a row now holds the totals of the wave's tokens
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) sh_u[w][h][cc * EPC + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h) { sh_m[w][h] = m[h]; sh_l[w][h] = l[h]; }
  }
  __syncthreads();

  // ---- merge the four waves -----------------------------------------------------
  const float vscale = KV == kFP8 ? a.v_scale[g] : 1.0f;
  const int P = a.num_parts;
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
    if (nparts == 1) {
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

// Split-KV reduce: one thread per (sequence, query head, column). Partition
// π left m_π (log2 domain), l_π and u_π; with m* = max m_π the output is
// Σ 2^(m_π − m*) u_π / Σ 2^(m_π − m*) l_π. Rows of sequences that fit in one
// partition were finished by the split kernel and are left alone.
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(MergeArgs a) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= a.total) return;
  const size_t row = idx / a.head_dim;
  const int d = (int)(idx % a.head_dim);
  const int b = (int)(row / a.hq);
  const int T = min(max(a.seq_lens[b], 0), min(a.max_seq_len, a.max_blocks * kBlockSize));
  const int nparts = (T + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;
  const int P = a.num_parts;
  const float* ml = a.ws_ml + row * P * 2;
  const float* u = a.ws_u + row * P * a.head_dim + d;
  float mt = -INFINITY;
  for (int pp = 0; pp < nparts; ++pp) mt = fmaxf(mt, ml[2 * pp]);
  float lt = 0.0f, ut = 0.0f;
  for (int pp = 0; pp < nparts; ++pp) {
    const float wgt = part_weight(ml[2 * pp], mt);
    lt = fmaf(wgt, ml[2 * pp + 1], lt);
    ut = fmaf(wgt, u[(size_t)pp * a.head_dim], ut);
  }
  a.out[idx] = lt > 0.0f ? ut / lt : 0.0f;
}

template <int KV, int DH, int HC>
hipError_t launch_t(const DecodeParams& p, const KernelArgs& a, hipStream_t s) {
  const size_t n = (size_t)p.batch * p.cache.num_kv_heads * a.num_chunks * p.num_parts;
  hipLaunchKernelGGL((decode_split_kernel<KV, DH, HC>), dim3((unsigned)n), dim3(kThreads), 0, s, a);
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

int decode_heads_per_wg(int group) {
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
  if (p.batch == 0) return hipSuccess;
  const int group = p.num_q_heads / p.cache.num_kv_heads;
  const int hc = decode_heads_per_wg(group);
  KernelArgs a;
  a.kc = static_cast<const uint8_t*>(p.cache.k);
  a.vc = static_cast<const uint8_t*>(p.cache.v);
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
  a.num_chunks = group / hc;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  const int dt = p.cache.dtype, dh = p.cache.head_dim;
  hipError_t e;
  if (dt == kF32) e = dh == 64 ? launch_hc<kF32, 64>(p, a, hc, s) : launch_hc<kF32, 128>(p, a, hc, s);
  else if (dt == kBF16) e = dh == 64 ? launch_hc<kBF16, 64>(p, a, hc, s) : launch_hc<kBF16, 128>(p, a, hc, s);
  else e = dh == 64 ? launch_hc<kFP8, 64>(p, a, hc, s) : launch_hc<kFP8, 128>(p, a, hc, s);
  if (e != hipSuccess || p.num_parts <= 1) return e;
  MergeArgs m;
  m.ws_ml = p.ws_ml;
  m.ws_u = p.ws_u;
  m.seq_lens = p.seq_lens;
  m.out = p.out;
  m.total = (size_t)p.batch * p.num_q_heads * dh;
  m.hq = p.num_q_heads;
  m.head_dim = dh;
  m.max_blocks = p.max_blocks;
  m.max_seq_len = p.max_seq_len;
  m.part_tokens = p.part_tokens;
  m.num_parts = p.num_parts;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((m.total + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, s, m);
  return hipGetLastError();
}

}  // namespace pkv
