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
// heads of that group, partition π of part_tokens tokens):
//   1. scores: each wave walks blocks π·P/16 + w, +4, …; a lane pairs with
//      three neighbours on one token row (quad), holds a quarter of that row
//      and the matching quarter of the HC queries, and a quad reduction yields
//      the HC scores of the token; scores go to LDS (log2 domain).
//   2. softmax statistics: workgroup max and sum per head over the partition;
//      scores are turned into p = 2^(s − m) in place.
//   3. values: each wave walks the same blocks; 16-byte V slices are read by
//      consecutive lanes (a row takes row_bytes/16 lanes) and accumulated as
//      fp32 p·v; lanes holding the same columns are summed at the end, then
//      the four waves through LDS.
//   4. if the sequence has one partition, o = u / l is written directly;
//      otherwise (m, l, u) go to the workspace, and the last workgroup of the
//      (b, g, chunk) to finish — found with a device-scope counter — merges
//      the partitions and resets the counter to zero.
// Masked slots (past the sequence end, or in a block whose id is out of the
// pool) are selected out, never multiplied by zero: pool slots may hold NaN.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <int KV, int DH>
struct Geometry {
  static constexpr int ESZ = KV == kF32 ? 4 : KV == kBF16 ? 2 : 1;  // stored bytes per element
  static constexpr int RB = DH * ESZ;        // bytes of one token row of one head
  static constexpr int EPC = 16 / ESZ;       // elements in a 16-byte slice
  static constexpr int NCH = RB / 64;        // score phase: 16-byte slices per lane (4 lanes a row)
  static constexpr int LPR = RB / 16;        // value phase: lanes per row
  static constexpr int RPI = kWave / LPR;    // value phase: rows per wave load
  static constexpr int NI = kBlockSize / RPI;  // value phase: loads per block
  // q registers per head and slice: packed bf16 pairs for bf16 and fp8 caches,
  // fp32 values for f32 caches
  static constexpr int QW = KV == kF32 ? 4 : KV == kBF16 ? 4 : 8;
  static_assert(RB % 64 == 0 && kWave % LPR == 0 && RPI <= kBlockSize, "unsupported row size");
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
  int32_t* ws_count;
  int num_blocks, hkv, hq, max_blocks, max_seq_len, part_tokens, num_parts, num_chunks;
  float scale_log2;  // scale · log2(e)
};

// Score contribution of one 16-byte K slice against one head's q slice.
template <int KV>
__device__ __forceinline__ float slice_dot(const uint32_t (&qs)[8], const uint4& k, float acc) {
  if constexpr (KV == kBF16) {
    acc = dot2_bf16(qs[0], k.x, acc);
    acc = dot2_bf16(qs[1], k.y, acc);
    acc = dot2_bf16(qs[2], k.z, acc);
    acc = dot2_bf16(qs[3], k.w, acc);
  } else if constexpr (KV == kF32) {
    acc = fmaf(__uint_as_float(qs[0]), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(qs[1]), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(qs[2]), __uint_as_float(k.z), acc);
    acc = fmaf(__uint_as_float(qs[3]), __uint_as_float(k.w), acc);
  } else {
    const uint32_t w[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = dot2_bf16(qs[2 * i], fp8x2_to_bf16x2<false>(w[i]), acc);
      acc = dot2_bf16(qs[2 * i + 1], fp8x2_to_bf16x2<true>(w[i]), acc);
    }
  }
  return acc;
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

template <int KV, int DH, int HC>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(KernelArgs a) {
  using G = Geometry<KV, DH>;
  extern __shared__ float smem[];

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
      for (int i = tid; i < HC * DH; i += kThreads)
        a.out[((size_t)b * a.hq + h0) * DH + i] = 0.0f;
    }
    return;
  }
  const int tok0 = part * a.part_tokens;
  const int ntok = min(a.part_tokens, T - tok0);
  const int nblk = (ntok + kBlockSize - 1) / kBlockSize;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks + tok0 / kBlockSize;
  const size_t head_stride = (size_t)kBlockSize * G::RB;     // bytes of one (block, head)

  float* logits = smem;                                       // [part_tokens][HC]
  float* red = smem + a.part_tokens * HC;                     // [kWaves][HC] scratch
  float* stats = red + kWaves * HC;                           // [2][HC]: m, l

  // ---- 1. scores ----------------------------------------------------------------
  {
    const int t = lane >> 2, j = lane & 3;
    uint32_t qreg[HC][G::NCH][8];
#pragma unroll
    for (int h = 0; h < HC; ++h) {
#pragma unroll
      for (int c = 0; c < G::NCH; ++c) {
        const int e0 = (c * 64 + j * 16) / G::ESZ;   // first element of this lane's slice
        if constexpr (KV == kF32) {
          const uint4 x = *reinterpret_cast<const uint4*>(
              static_cast<const float*>(a.q) + ((size_t)b * a.hq + h0 + h) * DH + e0);
          qreg[h][c][0] = x.x; qreg[h][c][1] = x.y; qreg[h][c][2] = x.z; qreg[h][c][3] = x.w;
        } else {
          const uint16_t* qp = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.hq + h0 + h) * DH + e0;
          const uint4 x = *reinterpret_cast<const uint4*>(qp);
          qreg[h][c][0] = x.x; qreg[h][c][1] = x.y; qreg[h][c][2] = x.z; qreg[h][c][3] = x.w;
          if constexpr (KV == kFP8) {
            const uint4 y = *reinterpret_cast<const uint4*>(qp + 8);
            qreg[h][c][4] = y.x; qreg[h][c][5] = y.y; qreg[h][c][6] = y.z; qreg[h][c][7] = y.w;
          }
        }
      }
    }
    float sc = a.scale_log2;
    if constexpr (KV == kFP8) sc *= a.k_scale[g];

    auto score_block = [&](int lb, const uint4 (&kv)[G::NCH], bool okb) {
      float s[HC];
#pragma unroll
      for (int h = 0; h < HC; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) acc = slice_dot<KV>(qreg[h][c], kv[c], acc);
        s[h] = quad_sum(acc);
      }
      const int tok = lb * kBlockSize + t;
      const bool valid = okb && tok < ntok;
#pragma unroll
      for (int h = 0; h < HC; ++h)
        if ((h & 3) == j) logits[tok * HC + h] = valid ? s[h] * sc : -INFINITY;
    };
    auto load_k = [&](int lb, uint4 (&kv)[G::NCH]) -> bool {
      const int phys = bt[lb];
      const bool okb = (unsigned)phys < (unsigned)a.num_blocks;
      if (okb) {
        const uint8_t* row = a.kc + ((size_t)phys * a.hkv + g) * head_stride + (size_t)t * G::RB + j * 16;
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) kv[c] = *reinterpret_cast<const uint4*>(row + c * 64);
      } else {
#pragma unroll
        for (int c = 0; c < G::NCH; ++c) kv[c] = make_uint4(0, 0, 0, 0);
      }
      return okb;
    };
    int lb = w;
    for (; lb + kWaves < nblk; lb += 2 * kWaves) {
      uint4 k0[G::NCH], k1[G::NCH];
      const bool o0 = load_k(lb, k0);
      const bool o1 = load_k(lb + kWaves, k1);
      score_block(lb, k0, o0);
      score_block(lb + kWaves, k1, o1);
    }
    if (lb < nblk) {
      uint4 k0[G::NCH];
      const bool o0 = load_k(lb, k0);
      score_block(lb, k0, o0);
    }
  }
  __syncthreads();

  // ---- 2. softmax statistics over the partition ------------------------------
  float m[HC], l[HC];
  {
    float mx[HC];
#pragma unroll
    for (int h = 0; h < HC; ++h) mx[h] = -INFINITY;
    for (int i = tid; i < ntok; i += kThreads) {
#pragma unroll
      for (int h = 0; h < HC; ++h) mx[h] = fmaxf(mx[h], logits[i * HC + h]);
    }
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      mx[h] = wave_max(mx[h]);
      if (lane == 0) red[w * HC + h] = mx[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      float v = red[h];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) v = fmaxf(v, red[ww * HC + h]);
      m[h] = v;   // finite: every partition holds at least one valid token
    }
    __syncthreads();
    float sm[HC];
#pragma unroll
    for (int h = 0; h < HC; ++h) sm[h] = 0.0f;
    for (int i = tid; i < ntok; i += kThreads) {
#pragma unroll
      for (int h = 0; h < HC; ++h) {
        const float p = fast_exp2(logits[i * HC + h] - m[h]);
        logits[i * HC + h] = p;
        sm[h] += p;
      }
    }
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      sm[h] = wave_sum(sm[h]);
      if (lane == 0) red[w * HC + h] = sm[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < HC; ++h) {
      float v = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) v += red[ww * HC + h];
      l[h] = v;
    }
  }

  // ---- 3. values -------------------------------------------------------------
  const int r = lane / G::LPR, cc = lane % G::LPR;
  float acc[HC][G::EPC];
#pragma unroll
  for (int h = 0; h < HC; ++h)
#pragma unroll
    for (int e = 0; e < G::EPC; ++e) acc[h][e] = 0.0f;

  for (int lb = w; lb < nblk; lb += kWaves) {
    const int phys = bt[lb];
    if ((unsigned)phys >= (unsigned)a.num_blocks) continue;
    const uint8_t* base = a.vc + ((size_t)phys * a.hkv + g) * head_stride + cc * 16;
    uint4 vv[G::NI];
#pragma unroll
    for (int i = 0; i < G::NI; ++i)
      vv[i] = *reinterpret_cast<const uint4*>(base + (size_t)(r + G::RPI * i) * G::RB);
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
      const int tok = lb * kBlockSize + r + G::RPI * i;
      if (tok < ntok) {
        float f[G::EPC];
        slice_values<KV, G::EPC>(vv[i], f);
        float p[HC];
#pragma unroll
        for (int h = 0; h < HC; ++h) p[h] = logits[tok * HC + h];
#pragma unroll
        for (int h = 0; h < HC; ++h)
#pragma unroll
          for (int e = 0; e < G::EPC; ++e) acc[h][e] = fmaf(p[h], f[e], acc[h][e]);
      }
    }
  }
  // lanes with the same columns (lane % LPR) hold partial sums of different rows
#pragma unroll
  for (int off = G::LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int e = 0; e < G::EPC; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, kWave);
  __syncthreads();  // all waves are done reading p from `logits`
  float* wsum = smem;  // [kWaves][HC][DH], reuses the score buffer
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < HC; ++h)
#pragma unroll
      for (int e = 0; e < G::EPC; ++e) wsum[(w * HC + h) * DH + cc * G::EPC + e] = acc[h][e];
  }
  __syncthreads();

  const float vscale = KV == kFP8 ? a.v_scale[g] : 1.0f;
  if (nparts == 1) {
    for (int i = tid; i < HC * DH; i += kThreads) {
      const int h = i / DH;
      float u = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) u += wsum[ww * HC * DH + i];
      float lh = 0.0f;
#pragma unroll
      for (int hh = 0; hh < HC; ++hh) if (hh == h) lh = l[hh];
      a.out[((size_t)b * a.hq + h0) * DH + i] = u * vscale / lh;
    }
    return;
  }

  // ---- 4. partials, then the last workgroup merges ----------------------------
  const int P = a.num_parts;
  for (int i = tid; i < HC * DH; i += kThreads) {
    const int h = i / DH, d = i % DH;
    float u = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) u += wsum[ww * HC * DH + i];
    a.ws_u[(((size_t)b * a.hq + h0 + h) * P + part) * DH + d] = u * vscale;
  }
  if (tid < HC) {
    float mh = 0.0f, lh = 0.0f;
#pragma unroll
    for (int hh = 0; hh < HC; ++hh) if (hh == tid) { mh = m[hh]; lh = l[hh]; }
    float* ml = a.ws_ml + (((size_t)b * a.hq + h0 + tid) * P + part) * 2;
    ml[0] = mh;
    ml[1] = lh;
  }
  __threadfence();  // make this partition's partials visible device-wide
  __syncthreads();
  __shared__ int is_last;
  if (tid == 0) {
    int32_t* counter = a.ws_count + ((size_t)b * a.hkv + g) * a.num_chunks + chunk;
    const int prev = atomicAdd(counter, 1);
    is_last = prev == nparts - 1;
    if (is_last) atomicExch(counter, 0);   // every partition has arrived: re-arm
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();  // see every other partition's partials

  for (int i = tid; i < HC * DH; i += kThreads) {
    const int h = i / DH, d = i % DH;
    const float* ml = a.ws_ml + ((size_t)b * a.hq + h0 + h) * P * 2;
    const float* u = a.ws_u + ((size_t)b * a.hq + h0 + h) * P * DH + d;
    float mt = -INFINITY;
    for (int pp = 0; pp < nparts; ++pp) mt = fmaxf(mt, __builtin_nontemporal_load(ml + 2 * pp));
    float lt = 0.0f, ut = 0.0f;
    for (int pp = 0; pp < nparts; ++pp) {
      const float wgt = fast_exp2(__builtin_nontemporal_load(ml + 2 * pp) - mt);
      lt = fmaf(wgt, __builtin_nontemporal_load(ml + 2 * pp + 1), lt);
      ut = fmaf(wgt, __builtin_nontemporal_load(u + (size_t)pp * DH), ut);
    }
    a.out[((size_t)b * a.hq + h0 + h) * DH + d] = ut / lt;
  }
}

template <int KV, int DH, int HC>
hipError_t launch_t(const DecodeParams& p, const KernelArgs& a, hipStream_t s) {
  const size_t score_floats = (size_t)p.part_tokens * HC + kWaves * HC + 2 * HC;
  const size_t sum_floats = (size_t)kWaves * HC * DH;
  const size_t lds = (score_floats > sum_floats ? score_floats : sum_floats) * sizeof(float);
  const size_t n = (size_t)p.batch * p.cache.num_kv_heads * a.num_chunks * p.num_parts;
  hipLaunchKernelGGL((decode_split_kernel<KV, DH, HC>), dim3((unsigned)n), dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <int KV, int DH>
hipError_t launch_hc(const DecodeParams& p, const KernelArgs& a, int hc, hipStream_t s) {
  switch (hc) {
    case 1: return launch_t<KV, DH, 1>(p, a, s);
    case 2: return launch_t<KV, DH, 2>(p, a, s);
    default: return launch_t<KV, DH, 4>(p, a, s);
  }
}

}  // namespace

int decode_heads_per_wg(int group) {
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
  a.ws_count = p.ws_count;
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
  if (dt == kF32) return dh == 64 ? launch_hc<kF32, 64>(p, a, hc, s) : launch_hc<kF32, 128>(p, a, hc, s);
  if (dt == kBF16) return dh == 64 ? launch_hc<kBF16, 64>(p, a, hc, s) : launch_hc<kBF16, 128>(p, a, hc, s);
  return dh == 64 ? launch_hc<kFP8, 64>(p, a, hc, s) : launch_hc<kFP8, 128>(p, a, hc, s);
}

}  // namespace pkv
