// Causal chunked prefill over a paged, cached prefix, on gfx950 MFMA.
//
// Method: "07｜KV Cache、FlashAttention与PagedAttention的内部过程", Q027 core
// answer and the FlashAttention section — attention is computed tile by tile
// with the scores and probabilities kept on chip, scale and mask fused, and
// the online softmax (running max m, sum l, weighted sum u, old statistics
// rescaled by exp(m_old − m_new)) gives the same result as the full softmax.
// "06 KV Cache…" 6.6 — prefill split into chunks; a chunk's queries see the
// cached prefix and the chunk's earlier tokens. Q025 table row 2 — the causal
// mask includes the diagonal.
//
// Workgroup = (sequence, KV head g, a chunk of GW ≤ 4 query heads of g, a tile
// of 64/GW queries), three streams of four waves: stream s takes key tiles
// s, s+3, s+6, … (three waves per SIMD, so each hides the others' latencies),
// and the streams' online-softmax states are merged into stream 0 at the end.
// When the query tiles alone give two or more workgroups per CU, each
// workgroup is one stream of four waves over all its keys instead, three
// workgroups to a CU, so their barriers do not hold one another back.
// Within a stream, wave w takes head w % GW and 16 queries. Keys go in tiles
// of 64 = four blocks; wave w of a stream gathers block w of its tiles:
//   * K and V of the block come in through raw buffer loads whose record limit
//     is the block's rows before the workgroup's last visible key (rows past it
//     and ids outside the pool read as zeros, with no memory access); the
//     stream's next tile's loads are in flight in registers while the current
//     tile is used, and its table entry is read a tile earlier still;
//   * K is stored row-major and padded, V transposed into groups of four keys
//     per column, so both feed MFMA operands with 16-byte LDS reads;
//   * Sᵀ = K·Qᵀ on MFMA 16x16x32 bf16 (keys are the M dimension, so each lane's
//     scores all belong to one query: lane % 16);
//   * the causal mask (select to −inf) is applied only on tiles that reach past
//     the wave's first query; online softmax in the log2 domain, with the scale
//     folded into the exponent; O is rescaled only when some query's running
//     max moved; the row sum stays lane-local until the end;
//   * Oᵀ += Vᵀ·Pᵀ on MFMA, keys ordered as the score layout left them, so no
//     shuffle of P is needed; P enters as a bf16 high part (truncated) plus the
//     bf16 rounding of the remainder (two MFMAs), which keeps the
//     probabilities to ~16 bits.
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "prefill_stream.h"

namespace pkv {

namespace {

constexpr int kStreamWaves = 4;                  // waves of one stream
// Workgroups of four waves (one stream) run three to a CU once the query
// tiles alone give at least this many (2 per CU); below it, one 12-wave
// workgroup per CU splits each query tile's keys over three streams.
constexpr int kOneStreamTiles = 2 * 256;
constexpr int kKeys = 64;                        // keys per tile
constexpr int kTileBlocks = kKeys / kBlockSize;  // blocks per tile, one per wave of a stream
static_assert(kTileBlocks == kStreamWaves, "one block of each key tile per wave");

struct Args {
  const uint8_t* kc;
  const uint8_t* vc;
  const uint16_t* q;
  const int32_t* q_start;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* out;
  int num_blocks, hkv, hq, max_blocks, num_qtiles, num_chunks;
  int unit_shift;   // log2(block_size / 16): a pool block holds 1, 2 or 4 16-row units
  float scale_log2;
};

// NS key streams of four waves share a workgroup: NS = 3, one workgroup per
// CU with its streams merged through LDS at the end; NS = 1, four-wave
// workgroups, three per CU, each on its own barrier schedule.
template <int DH, int GW, int NS>
__global__ __launch_bounds__(NS * kStreamWaves * kWave) void prefill_kernel(Args a) {
  constexpr int kStreams = NS;
  constexpr int QT = 64 / GW;              // queries per workgroup
  constexpr int KROW = DH + 16;            // padded K row in LDS (elements; +16 measured fewest conflicts)
  constexpr int NDC = DH / 32;             // 32-wide k-steps for Q·Kᵀ
  constexpr int NDT = DH / 16;             // 16-row output tiles of Oᵀ
  constexpr int CPR = DH / 8;              // 16-byte chunks per row
  constexpr int RB = DH * 2;               // bytes of one token row of one head
  constexpr int NKL = kBlockSize * CPR / kWave;    // K chunks per lane per block
  constexpr int NVL = kBlockSize / 4 * CPR;        // lanes that gather V (4 rows each)
  // V in LDS: [key quad][column][4 keys] bf16, 8 bytes per (quad, column),
  // with 16 bytes of padding after every 8 columns (the transposing stores
  // of neighbouring lanes are 64 bytes apart without it) and 128 bytes after
  // every quad (the PV operand reads of lanes 0-15 and 16-31 use neighbouring
  // quads; an odd multiple of 128 bytes puts them in opposite bank halves)
  constexpr int VCOL = 4;                               // elements per (quad, column)
  constexpr int VQ = DH * VCOL + (DH / 8) * 8 + 64;     // elements per key quad
  __shared__ __attribute__((aligned(16))) uint16_t k_lds_all[kStreams][kKeys * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds_all[kStreams][(kKeys / 4) * VQ];
  auto v_index = [](int kq, int d) { return kq * VQ + d * VCOL + (d / 8) * 8; };

  const uint32_t L = xcd_logical_index(flat_block_id(), flat_grid_size());
  const int qtile = L % a.num_qtiles;
  const int chunk = (L / a.num_qtiles) % a.num_chunks;
  const int g = (L / a.num_qtiles / a.num_chunks) % a.hkv;
  const int s = L / a.num_qtiles / a.num_chunks / a.hkv;

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
  const int stream = wave / kStreamWaves;                  // 0: even key tiles, 1: odd ones
  const int w = wave % kStreamWaves;                       // wave within the stream
  uint16_t* k_lds = k_lds_all[stream];
  uint16_t* v_lds = v_lds_all[stream];
  const int q_lo = __builtin_amdgcn_readfirstlane(a.q_start[s]);
  const int C = __builtin_amdgcn_readfirstlane(a.q_start[s + 1]) - q_lo;   // queries of this sequence
  const int T = __builtin_amdgcn_readfirstlane(min(a.seq_lens[s], (a.max_blocks << a.unit_shift) * kBlockSize));
  if (qtile * QT >= C || T <= 0) return;
  const int base_pos = T - C;                             // position of query 0
  const int group = a.hq / a.hkv;
  const int head = g * group + chunk * GW + (w % GW);
  const int qi0 = qtile * QT + (w / GW) * 16;             // this wave's first query
  const int col = lane & 15, kg = lane >> 4;
  const int my_q = qi0 + col;                             // query whose scores this lane holds
  const bool q_valid = my_q < C;
  const int my_pos = q_valid ? base_pos + my_q : T - 1;
  const int wave_first_pos = base_pos + qi0;              // smallest position of the wave's queries
  // last key any query of this workgroup sees
  const int wg_last_q = min(C, qtile * QT + QT) - 1;
  const int kend = min(T, base_pos + wg_last_q + 1);
  const int ntiles = (kend + kKeys - 1) / kKeys;
  const int32_t* bt = a.block_tables + (size_t)s * a.max_blocks;
  // 16-row unit u is rows (u mod 2^shift)·16 … of pool block entry u >> shift
  const int unit_mask = (1 << a.unit_shift) - 1;
  const size_t head_stride = ((size_t)kBlockSize * RB) << a.unit_shift;   // bytes of one (pool block, head)

  // Qᵀ operand: lane holds Q[my_q][dc*32 + kg*8 .. +7]
  bf16x8_t qreg[NDC];
  {
    const int qrow = q_lo + (q_valid ? my_q : 0);
    const uint16_t* qp = a.q + ((size_t)qrow * a.hq + head) * DH + kg * 8;
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
      qreg[dc] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + dc * 32));
  }

  f32x4_t o[NDT];
#pragma unroll
  for (int i = 0; i < NDT; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;   // m in raw-score units

  // ---- gathers: wave w takes block w of each tile -------------------------------
  // K: lane loads rows lane/CPR + (64/CPR)·i, chunk lane % CPR.
  // V: lane < NVL loads rows 4·(lane/CPR) … +3 of chunk lane % CPR.
  const int k_off = (lane / CPR) * RB + (lane % CPR) * 16;
  const int v_off = (lane / CPR) * 4 * RB + (lane % CPR) * 16;
  struct Stage {
    uint4 k[NKL], v[4];
  };
  auto table_entry = [&](int kt) -> int {
    const int lb = kt * kTileBlocks + w;
    return lb * kBlockSize < kend ? __builtin_amdgcn_readfirstlane(bt[lb >> a.unit_shift]) : -1;
  };
  // bit b set: block b of key tile kt names a pool block (an id outside the
  // pool, or −1, reads as zeros and its keys must be masked, not scored 0)
  auto tile_valid = [&](int kt) -> int {
    int mask = 0;
#pragma unroll
    for (int b = 0; b < kTileBlocks; ++b) {
      const int lb = kt * kTileBlocks + b;
      const int phys = lb * kBlockSize < kend ? __builtin_amdgcn_readfirstlane(bt[lb >> a.unit_shift]) : 0;
      mask |= ((unsigned)phys < (unsigned)a.num_blocks) << b;
    }
    return mask;
  };
  auto fetch = [&](int kt, int phys, Stage& st) {
    const int rows = min(kBlockSize, max(0, kend - (kt * kTileBlocks + w) * kBlockSize));
    const bool ok = (unsigned)phys < (unsigned)a.num_blocks;
    const int unit_row0 = ((kt * kTileBlocks + w) & unit_mask) * kBlockSize;
    const size_t off = ((size_t)(ok ? phys : 0) * a.hkv + g) * head_stride + (size_t)unit_row0 * RB;
    const int records = __builtin_amdgcn_readfirstlane(ok ? rows * RB : 0);
    const auto rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.kc + off), 0, records, kBufferRsrcWord3);
    const auto rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.vc + off), 0, records, kBufferRsrcWord3);
#pragma unroll
    for (int i = 0; i < NKL; ++i) st.k[i] = buffer_load16(rk, k_off + i * (kWave / CPR) * RB);
    if (lane < NVL) {
#pragma unroll
      for (int r = 0; r < 4; ++r) st.v[r] = buffer_load16(rv, v_off + r * RB);
    }
  };
  auto store = [&](const Stage& st) {
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const int key = w * kBlockSize + lane / CPR + i * (kWave / CPR);
      *reinterpret_cast<uint4*>(&k_lds[key * KROW + (lane % CPR) * 8]) = st.k[i];
    }
    if (lane < NVL) {
      const int kq = w * (kBlockSize / 4) + lane / CPR, ch = lane % CPR;
      const uint32_t rw[4][4] = {{st.v[0].x, st.v[0].y, st.v[0].z, st.v[0].w},
                                 {st.v[1].x, st.v[1].y, st.v[1].z, st.v[1].w},
                                 {st.v[2].x, st.v[2].y, st.v[2].z, st.v[2].w},
                                 {st.v[3].x, st.v[3].y, st.v[3].z, st.v[3].w}};
#pragma unroll
      for (int e = 0; e < 4; ++e) {       // dword e holds columns 2e (low) and 2e+1 (high)
        const uint32_t lo01 = __builtin_amdgcn_perm(rw[1][e], rw[0][e], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(rw[3][e], rw[2][e], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(rw[1][e], rw[0][e], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(rw[3][e], rw[2][e], 0x07060302u);
        const int d = ch * 8 + 2 * e;
        *reinterpret_cast<uint2*>(&v_lds[v_index(kq, d)]) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(&v_lds[v_index(kq, d + 1)]) = make_uint2(hi01, hi23);
      }
    }
  };

  // ---- one tile's work on the K/V tile in LDS -----------------------------------
  auto compute = [&](int kt) {
    const int key0 = kt * kKeys;
    // Sᵀ = K·Qᵀ: four 16-key tiles
    f32x4_t st[4];
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const bf16x8_t kk = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4*>(&k_lds[(t4 * 16 + col) * KROW + dc * 32 + kg * 8]));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qreg[dc], acc, 0, 0, 0);
      }
      st[t4] = acc;
    }
    // inclusive causal mask, only where the tile reaches past the wave's
    // first query, and the keys of blocks outside the pool
    const int valid = tile_valid(kt);
    if (key0 + kKeys - 1 > wave_first_pos || valid != (1 << kTileBlocks) - 1) {
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + t4 * 16 + kg * 4 + i > my_pos || !((valid >> t4) & 1)) st[t4][i] = -INFINITY;
    }
    // online softmax: the lane's 16 scores all belong to query my_q
    float mt = fmaxf(fmaxf(st[0][0], st[0][1]), fmaxf(st[0][2], st[0][3]));
#pragma unroll
    for (int t4 = 1; t4 < 4; ++t4)
      mt = fmaxf(mt, fmaxf(fmaxf(st[t4][0], st[t4][1]), fmaxf(st[t4][2], st[t4][3])));
    mt = pair_halves32(pair_rows16(mt, MaxOp()), MaxOp());
    // m stays −inf while every key a query has met is masked (a later
    // stream's first tile can lie wholly after an early query): the old state is then
    // empty (weight 0) and the masked scores give p = 0
    const float m_new = fmaxf(m_run, mt);
    if (__any(m_new > m_run)) {                           // rescale only when a max moved
      const float alpha = m_run == -INFINITY ? 0.0f : fast_exp2((m_run - m_new) * a.scale_log2);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run == -INFINITY ? 0.0f : m_run * a.scale_log2;
    float psum = 0.0f;
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(fmaf(st[t4][i], a.scale_log2, -mc));
        st[t4][i] = p;
        psum += p;
      }
    l_run += psum;

    // Oᵀ += Vᵀ·Pᵀ over two 32-key steps; P = hi + lo with hi the truncated
    // bf16 of p and lo the bf16 rounding of p − hi, both through the MFMA (V is
    // exact in bf16, so the product keeps ~16-bit probabilities instead of
    // bf16's 2^-9 relative rounding)
#pragma unroll
    for (int kc2 = 0; kc2 < 2; ++kc2) {
      float pv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) { pv[i] = st[2 * kc2][i]; pv[4 + i] = st[2 * kc2 + 1][i]; }
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
      const int quad_a = (2 * kc2) * 4 + kg;              // keys (2kc2)*16 + kg*4 .. +3
      const int quad_b = (2 * kc2 + 1) * 4 + kg;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int d = dt * 16 + col;
        const uint2 va = *reinterpret_cast<const uint2*>(&v_lds[v_index(quad_a, d)]);
        const uint2 vb = *reinterpret_cast<const uint2*>(&v_lds[v_index(quad_b, d)]);
        const bf16x8_t vv = __builtin_bit_cast(bf16x8_t, make_uint4(va.x, va.y, vb.x, vb.y));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, p_hi, o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, p_lo, o[dt], 0, 0, 0);
      }
    }
  };

  // Stream s takes tiles s, s+3, …, each stream with its own LDS tile and its
  // next tile's loads in flight in registers; table entries are read a tile
  // ahead of their gathers. All streams meet at every barrier.
  {
    Stage st;
    int kt = stream;
    fetch(kt, table_entry(kt), st);
    int pn = table_entry(kt + kStreams);
    const int iters = (ntiles + kStreams - 1) / kStreams;
    for (int it = 0; it < iters; ++it, kt += kStreams) {
      const bool active = kt < ntiles;
      if (active) store(st);
      __syncthreads();
      if (kt + kStreams < ntiles) {
        fetch(kt + kStreams, pn, st);
        pn = table_entry(kt + 2 * kStreams);
      }
      if (active) compute(kt);
      __syncthreads();
    }
  }

  // ---- merge the other streams into stream 0 through LDS, one per round ----
  // Each lane of a stream-r wave leaves m, its partial l and its 4·NDT output
  // values; the stream-0 wave holding the same queries and head folds them in.
  {
    float* xch = reinterpret_cast<float*>(&k_lds_all[0][0]);
    constexpr int NX = 2 + 4 * NDT;                        // floats per lane
    static_assert(NS == 1 || kStreamWaves * kWave * NX * 4 <= (int)sizeof(k_lds_all), "merge area");
    float* mine = xch + ((size_t)w * kWave + lane) * NX;
#pragma unroll
    for (int r = 1; r < kStreams; ++r) {
      if (stream == r) {
        mine[0] = m_run;
        mine[1] = l_run;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) mine[2 + 4 * dt + j] = o[dt][j];
      }
      __syncthreads();
      if (stream == 0) {
        const float m1 = mine[0];
        const float mt = fmaxf(m_run, m1);                 // −inf only if neither saw a valid key
        const float a0 = m_run == -INFINITY ? 0.0f : fast_exp2((m_run - mt) * a.scale_log2);
        const float a1 = m1 == -INFINITY ? 0.0f : fast_exp2((m1 - mt) * a.scale_log2);
        l_run = a0 * l_run + a1 * mine[1];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) o[dt][j] = a0 * o[dt][j] + a1 * mine[2 + 4 * dt + j];
        m_run = mt;
      }
      __syncthreads();
    }
    if (stream != 0) return;
  }

  // ---- finish: l over the four lanes of a query, o = u / l ----
  const float lt = pair_halves32(pair_rows16(l_run, AddOp()), AddOp());
  if (!q_valid) return;
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;   // no valid key at all: zeros
  float* op = a.out + ((size_t)(q_lo + my_q) * a.hq + head) * DH + kg * 4;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    const f32x4_t r = o[dt] * inv;
    *reinterpret_cast<float4*>(op + dt * 16) = make_float4(r[0], r[1], r[2], r[3]);
  }
}

template <int DH, int NS>
hipError_t launch_gw(Args a, size_t n, int gw, hipStream_t s) {
  const dim3 grid((unsigned)n), block(NS * kStreamWaves * kWave);
  switch (gw) {
    case 1: hipLaunchKernelGGL((prefill_kernel<DH, 1, NS>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<DH, 2, NS>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((prefill_kernel<DH, 4, NS>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

template <int DH>
hipError_t launch_dh(const PrefillParams& p, Args a, int gw, hipStream_t s) {
  const size_t n = (size_t)p.num_seqs * a.hkv * a.num_chunks * a.num_qtiles;
  return n >= (size_t)kOneStreamTiles ? launch_gw<DH, 1>(a, n, gw, s) : launch_gw<DH, 3>(a, n, gw, s);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, hipStream_t s) {
  if (p.num_seqs == 0 || p.max_q_len == 0) return hipSuccess;
  const int group = p.num_q_heads / p.cache.num_kv_heads;
  const int gw = group >= 4 ? 4 : group;     // group is 1, 2 or a multiple of 4
  Args a;
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
  a.num_chunks = group / gw;
  a.num_qtiles = (p.max_q_len + (64 / gw) - 1) / (64 / gw);
  a.unit_shift = __builtin_ctz((unsigned)p.cache.block_size / kBlockSize);
  a.scale_log2 = p.scale * 1.4426950408889634f;
  return p.cache.head_dim == 64 ? launch_dh<64>(p, a, gw, s) : launch_dh<128>(p, a, gw, s);
}

// ===========================================================================
// Key-stream form: the body is in prefill_stream.h.
namespace {

template <int DH, int RG, bool B8>
__global__ __launch_bounds__(8 * kWave, 1) void prefill_stream_kernel(SArgs a) {
  constexpr int NS = StreamShape<RG>::NS;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[stream_lds_bytes<DH, NS, RG>()];
  prefill_stream_body<DH, NS, RG, B8>(a, lds, xcd_logical_index(flat_block_id(), flat_grid_size()));
}

// (B8: pools of 8-token blocks)
template <int DH, int RG>
hipError_t launch_stream_dh(const PrefillParams& p, hipStream_t s) {
  const SArgs a = make_sargs(p, StreamShape<RG>::ROWS);
  const size_t n = stream_workgroups(p, a);
  if (p.cache.block_size == kBlockSize / 2)
    hipLaunchKernelGGL((prefill_stream_kernel<DH, RG, true>), dim3((unsigned)n), dim3(8 * kWave), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_stream_kernel<DH, RG, false>), dim3((unsigned)n), dim3(8 * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_stream(const PrefillParams& p, int rows, hipStream_t s) {
  if (p.num_seqs == 0 || p.max_q_len == 0) return hipSuccess;
  if (rows == 256 && p.cache.head_dim == 128) return launch_stream_dh<128, 8>(p, s);
  if (rows >= 128) return p.cache.head_dim == 64 ? launch_stream_dh<64, 4>(p, s) : launch_stream_dh<128, 4>(p, s);
  return p.cache.head_dim == 64 ? launch_stream_dh<64, 2>(p, s) : launch_stream_dh<128, 2>(p, s);
}

}  // namespace pkv
