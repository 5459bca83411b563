// Device helpers shared by the gfx950 kernels: bf16/fp8 unpacking, DPP and
// wave reductions, and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlockSize = 16;   // the kernels' unit of 16 token rows (a pool block of bs holds bs/16)
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kNumXcd = 8;       // MI355X: 8 accelerator dies, each with its own L2

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// bf16 pair packed in a dword: element 0 in the low half.
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// a.x*b.x + a.y*b.y + c on two packed bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two OCP e4m3 bytes of a dword (low pair when hi == false) → packed bf16
// pair; exact, since every e4m3 value is a bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Two OCP e4m3 bytes → two fp32 (exact).
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// OCP e4m3fn encode, round to nearest even, saturating at ±448, NaN kept.
// Integer formulation on the fp32 bit pattern (the round-half-even carry
// trick on the 3 kept mantissa bits); subnormal outputs use the exact
// scaling by 2^9 followed by an ties-to-even integer rounding.
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;            // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;           // >= 448 (and inf): saturate
  if (a < 0x3c800000u) {                               // below 2^-6: spacing 2^-9
    const float q = __builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)q;                         // 0..8; 8 is the first normal
  }
  // keep 3 mantissa bits with ties to even
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) & 0xfff00000u;
  const int e = (int)(r >> 23) - 127;                  // -6 … 8 (9 only past 448)
  const uint32_t m = (r >> 20) & 7u;
  uint32_t code = ((uint32_t)(e + 7) << 3) | m;
  if (code > 0x7eu) code = 0x7eu;
  return sign | code;
}

// Lane exchange inside a row of 16 lanes (DPP).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;      // lane i of a 16-lane row reads lane 15 - i
constexpr int kRowHalfMirror = 0x141;  // lane i of an 8-lane half-row reads lane 7 - i
constexpr int kRowRor4 = 0x124;        // rotate each 16-lane row by 4 lanes
constexpr int kRowRor8 = 0x128;        // rotate each 16-lane row by 8 lanes

// Cross-row exchanges on gfx950's lane-swap instructions (VALU, no LDS
// round trip). pair_rows16: op(x of this 16-lane row, x of its partner row:
// rows 0↔1 and 2↔3); pair_halves32: op(x of lanes 0-31, x of lanes 32-63).
// Both lanes of a pair evaluate op on the same operands in the same order,
// so they receive the same bits.
template <typename Op>
__device__ __forceinline__ float pair_rows16(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <typename Op>
__device__ __forceinline__ float pair_halves32(float x, Op op) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
struct MaxOp {
  __device__ float operator()(float x, float y) const { return fmaxf(x, y); }
};
struct AddOp {
  __device__ float operator()(float x, float y) const { return x + y; }
};

// Raw buffer loads: a resource names a base address and a byte limit; a load
// at or past the limit returns zeros and makes no memory access.
constexpr int kBufferRsrcWord3 = 0x00020000;   // gfx9 raw-buffer format word
constexpr int kCacheNonTemporal = 2;            // cache-policy operand: nt

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int offset) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i x = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
  return make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
}

// The same load with the non-temporal hint, for data read exactly once.
__device__ __forceinline__ uint4 buffer_load16_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i x = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, kCacheNonTemporal);
  return make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
}

// 8- and 4-byte forms of the non-temporal load.
__device__ __forceinline__ uint2 buffer_load8_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i x = __builtin_amdgcn_raw_buffer_load_b64(r, offset, 0, kCacheNonTemporal);
  return make_uint2((uint32_t)x[0], (uint32_t)x[1]);
}

__device__ __forceinline__ uint32_t buffer_load4_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, offset, 0, kCacheNonTemporal);
}

// 16-, 8- or 4-byte raw buffer load with cache-policy operand AUX (0, or
// kCacheNonTemporal for data read exactly once).
template <int AUX>
__device__ __forceinline__ uint4 buffer_load16_aux(__amdgpu_buffer_rsrc_t r, int offset) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i x = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, AUX);
  return make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
}

template <int AUX>
__device__ __forceinline__ uint2 buffer_load8_aux(__amdgpu_buffer_rsrc_t r, int offset) {
  typedef int v2i __attribute__((ext_vector_type(2)));
  const v2i x = __builtin_amdgcn_raw_buffer_load_b64(r, offset, 0, AUX);
  return make_uint2((uint32_t)x[0], (uint32_t)x[1]);
}

template <int AUX>
__device__ __forceinline__ uint32_t buffer_load4_aux(__amdgpu_buffer_rsrc_t r, int offset) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, offset, 0, AUX);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Hardware hands consecutive workgroup ids to the XCDs round-robin. This
// returns a logical work index such that a contiguous range of logical
// indices runs on one XCD (and shares its L2): id → (id % 8) * (n / 8) + id / 8,
// applied when the grid divides evenly, identity otherwise.
__device__ __forceinline__ uint32_t xcd_logical_index(uint32_t id, uint32_t n) {
  if (n % kNumXcd != 0) return id;
  return (id % kNumXcd) * (n / kNumXcd) + id / kNumXcd;
}

// The same idea at a coarser grain, for work whose neighbours in a batch may
// differ in size: consecutive logical indices come in groups of c that share
// data (say, the workgroups of a few KV heads of one sequence); each group
// stays on one XCD, and the groups are dealt to the XCDs in turn, so a run of
// large groups in the batch spreads over all eight. Ids past the last whole
// round of 8·c groups keep the hardware order. A bijection on [0, n).
__device__ __forceinline__ uint32_t grouped_xcd_index(uint32_t id, uint32_t n, uint32_t c) {
  const uint32_t full = n / (kNumXcd * c) * (kNumXcd * c);
  if (id >= full) return id;
  const uint32_t x = id % kNumXcd, s = id / kNumXcd;
  return ((s / c) * kNumXcd + x) * c + s % c;
}

__device__ __forceinline__ uint32_t flat_block_id() {
  return blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
}

__device__ __forceinline__ uint32_t flat_grid_size() { return gridDim.x * gridDim.y * gridDim.z; }

}  // namespace pkv
