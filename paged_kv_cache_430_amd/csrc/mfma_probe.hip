// Matrix-core rate probe: the bf16 MFMA rate this GPU sustains with every
// compute unit busy, for the product pattern of the chunked prefill's steady
// iteration and nothing else (no memory traffic, no vector work).
//
// The prefill computes its tiles' Sᵀ = K·Qᵀ and Oᵀ += Vᵀ·Pᵀ on
// v_mfma_f32_32x32x16_bf16 ("07｜KV Cache、FlashAttention与PagedAttention的内部
// 过程", the FlashAttention section: tiles kept on chip, the products done
// tile by tile). Its steady iteration issues, per wave, 16 PV products on four
// accumulators and 8 Sᵀ products on a fifth, Sᵀ alternating with PV in the
// second half. This kernel issues exactly that sequence, `iterations` times,
// from 8 waves per workgroup (two per SIMD, as the prefill runs), so its rate
// is the ceiling the prefill's matrix-core throughput is measured against:
// the published peak assumes a clock the chip does not hold under a full
// matrix-core load.
//
// Operands: lane l of every wave reads bf16 elements [8(l + j), 8(l + j) + 8)
// of `operands` for operand j < 20, so the kernel reads the first
// kMfmaProbeOperands values. Each lane writes the sum of its five
// accumulators' 80 values to sink[64·(8·wg + wave) + lane].
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kMfmaProbeWaves = 8;
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;

__global__ __launch_bounds__(kMfmaProbeWaves * kWave) void mfma_rate_kernel(const uint16_t* operands,
                                                                            int iterations, float* sink) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  bf16x8_t opnd[20];
#pragma unroll
  for (int j = 0; j < 20; ++j)
    opnd[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(operands + 8 * (lane + j)));
  f32x16_t o[4] = {}, acc = {};
  for (int it = 0; it < iterations; ++it) {
#pragma unroll
    for (int k = 0; k < 24; ++k) {
      if (k < 4) {
        o[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k], opnd[16], o[k], 0, 0, 0);
      } else if (k < 8) {
        o[k - 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[k - 4], opnd[17], o[k - 4], 0, 0, 0);
      } else {
        const int h = (k - 8) >> 1 & 3;
        const bool pv = ((k - 8) & 1) == 0;
        if (pv)
          o[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[4 + h], opnd[k < 16 ? 18 : 19], o[h], 0, 0, 0);
        else
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opnd[8 + (k < 16 ? 0 : 4) + h], opnd[12 + h], acc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);     // keep the prefill's order
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += o[0][r] + o[1][r] + o[2][r] + o[3][r] + acc[r];
  sink[((size_t)blockIdx.x * kMfmaProbeWaves + w) * kWave + lane] = s;
}

// The prefill's steady iteration with its data movement but without its
// arithmetic dependences, per wave and iteration: the same 24 products (16
// PV on four accumulators with a high and a low P operand, 8 Sᵀ on a fifth),
// 96 vector FMAs and 16 exponentials over the Sᵀ results (the softmax's
// vector work), and
//   MODE ≥ 1: the operands read from LDS as the prefill reads them — 8
//             ds_read_b128 of a K tile and 16 transposing 8-byte reads of a V
//             tile (16 KiB per wave, 128 KiB per workgroup);
//   MODE 2:   also the tile stream: 8 LDS-direct loads of 1 KiB per wave
//             (64 KiB per workgroup, the K and V tiles of four streams) into
//             a second LDS region, a wait for them and a workgroup barrier.
// The read region [0, 64 KiB) is filled from `tiles` at the start (N(0,1)
// values keep the matrix cores at the prefill's power); tile loads read
// 1 KiB units of the first MiB of `tiles`, the K and V tiles of an
// iteration sit at rotating 8 KiB offsets of the read region. Each lane
// writes the sum of its accumulators and vector values to
// sink[512·wg + thread].
constexpr int kMixTilesBytes = 1 << 20;

template <int MODE>
__global__ __launch_bounds__(kMfmaProbeWaves * kWave) void prefill_mix_kernel(const uint16_t* operands,
                                                                              const uint8_t* tiles, int iterations,
                                                                              float* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t sh[128 * 1024];
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int i = threadIdx.x; i < 64 * 1024 / 16; i += kMfmaProbeWaves * kWave)
    reinterpret_cast<uint4*>(sh)[i] = reinterpret_cast<const uint4*>(tiles)[i];
  __syncthreads();
  bf16x8_t q[8], p[2], plo[2];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    q[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(operands + 8 * (lane + j)));
  p[0] = q[0]; p[1] = q[1]; plo[0] = q[2]; plo[1] = q[3];
  f32x16_t o[4] = {}, acc = {};
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = __uint_as_float(0x3f800000u | (uint32_t)(lane * 16 + i) << 8);   // [1, 2)
  const float ca = 0.5f, cb = 0.25f;
  i32x4_t rsrc;
  rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)tiles);
  rsrc[1] = __builtin_amdgcn_readfirstlane((int)((uint64_t)(uintptr_t)tiles >> 32) & 0xffff);
  rsrc[2] = kMixTilesBytes;
  rsrc[3] = kBufferRsrcWord3;
  const int stream = w >> 1;
  for (int it = 0; it < iterations; ++it) {
    bf16x8_t v[4][2], k[8];
    if constexpr (MODE >= 1) {
      const int kb = ((it * 3 + stream) & 7) * 8192, vb = ((it * 5 + stream + 4) & 7) * 8192;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const uint8_t* base = sh + vb + dt * 2048 + ks * 1024 + lane * 8;
          const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_u8*)base));
          const uint2 hi =
              __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_u8*)(base + 512)));
          v[dt][ks] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
      for (int j = 0; j < 8; ++j) k[j] = *reinterpret_cast<const bf16x8_t*>(sh + kb + j * 1024 + lane * 16);
    } else {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) { v[dt][0] = q[dt]; v[dt][1] = q[dt + 4]; }
#pragma unroll
      for (int j = 0; j < 8; ++j) k[j] = q[(j + 3) & 7];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[dt][ks], p[ks], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[dt][ks], plo[ks], o[dt], 0, 0, 0);
      }
    acc = f32x16_t{};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[j], q[j], acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 96; ++i) x[i & 15] = fmaf(x[i & 15], ca, cb * acc[i & 15]);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = fast_exp2(fminf(x[i], 64.0f));
    p[0] = __builtin_bit_cast(bf16x8_t, make_uint4(__float_as_uint(x[0]) >> 16 | (__float_as_uint(x[1]) & 0xffff0000u),
                                                   __float_as_uint(x[2]) >> 16 | (__float_as_uint(x[3]) & 0xffff0000u),
                                                   __float_as_uint(x[4]) >> 16 | (__float_as_uint(x[5]) & 0xffff0000u),
                                                   __float_as_uint(x[6]) >> 16 | (__float_as_uint(x[7]) & 0xffff0000u)));
    p[1] = __builtin_bit_cast(bf16x8_t, make_uint4(__float_as_uint(x[8]) >> 16 | (__float_as_uint(x[9]) & 0xffff0000u),
                                                   __float_as_uint(x[10]) >> 16 | (__float_as_uint(x[11]) & 0xffff0000u),
                                                   __float_as_uint(x[12]) >> 16 | (__float_as_uint(x[13]) & 0xffff0000u),
                                                   __float_as_uint(x[14]) >> 16 | (__float_as_uint(x[15]) & 0xffff0000u)));
    if constexpr (MODE >= 2) {
      // 8 KiB per wave into [64 KiB, 128 KiB): 1 KiB pieces w·8 … w·8+7
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int piece = w * 8 + i;
        const int vo = ((it * 64 + piece) & (kMixTilesBytes / 1024 - 1)) * 1024 + lane * 16;
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen offset:0 lds"
                     :
                     : "v"(vo), "s"((uint32_t)(uintptr_t)(lds_u8*)(sh + 65536 + piece * 1024)), "s"(rsrc)
                     : "memory");
      }
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      __syncthreads();
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += o[0][r] + o[1][r] + o[2][r] + o[3][r] + acc[r] + x[r];
  sink[(size_t)blockIdx.x * kMfmaProbeWaves * kWave + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_prefill_mix(const void* operands, const void* tiles, int mode, int iterations, int num_wgs,
                              float* sink, hipStream_t s) {
  const auto* op = static_cast<const uint16_t*>(operands);
  const auto* t = static_cast<const uint8_t*>(tiles);
  const dim3 grid((unsigned)num_wgs), block(kMfmaProbeWaves * kWave);
  if (mode == 0) hipLaunchKernelGGL(prefill_mix_kernel<0>, grid, block, 0, s, op, t, iterations, sink);
  else if (mode == 1) hipLaunchKernelGGL(prefill_mix_kernel<1>, grid, block, 0, s, op, t, iterations, sink);
  else hipLaunchKernelGGL(prefill_mix_kernel<2>, grid, block, 0, s, op, t, iterations, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_rate(const void* operands, int iterations, int num_wgs, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)num_wgs), dim3(kMfmaProbeWaves * kWave), 0, s,
                     static_cast<const uint16_t*>(operands), iterations, sink);
  return hipGetLastError();
}

}  // namespace pkv
