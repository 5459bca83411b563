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

}  // namespace

hipError_t launch_mfma_rate(const void* operands, int iterations, int num_wgs, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)num_wgs), dim3(kMfmaProbeWaves * kWave), 0, s,
                     static_cast<const uint16_t*>(operands), iterations, sink);
  return hipGetLastError();
}

}  // namespace pkv
