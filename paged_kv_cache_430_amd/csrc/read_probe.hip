// Streaming-read probe: the HBM read rate this GPU sustains for the access
// pattern of paged decode, with no arithmetic beyond folding the bytes.
//
// Paged decode streams 4 KiB (block, head) tiles (16 rows of 256 bytes for a
// bf16 cache at Dh = 128) through a block table ("07｜KV Cache、FlashAttention
// 与PagedAttention的内部过程", Q028; "06 KV Cache…" 6.5: blocks sit anywhere in
// the pool and the table says where). This kernel reads the same tiles with
// the same raw buffer loads and the non-temporal hint, in whatever order a
// list of tile ids gives: in order for a contiguous stream, a permutation for
// the scattered order of a real pool. Its rate is the ceiling the decode's
// achieved bandwidth is measured against.
//
// Workgroup i of G takes ids [i·n/G, (i+1)·n/G); its 8 waves take every 8th
// tile of that range, four tiles (16 KiB) in flight per wave. Each wave holds
// 64 upcoming ids, one per lane, loaded a round ahead and read back with lane
// reads, so the id list adds no dependent latency. The XOR of every dword a
// workgroup read goes to sink[i], which keeps the loads live and lets a test
// check that exactly the listed tiles were read.
#include "device_common.h"
#include "launch.h"

namespace pkv {

namespace {

constexpr int kProbeWaves = 8;
constexpr int kTileBytes = 4096;
constexpr int kLoadsPerTile = kTileBytes / (kWave * 16);   // 16-byte loads per lane per tile
constexpr int kInFlight = 4;                                // tiles in flight per wave

__global__ __launch_bounds__(kProbeWaves * kWave) void stream_read_kernel(const uint8_t* buf, int64_t buf_tiles,
                                                                          const int32_t* ids, int n_tiles,
                                                                          uint32_t* sink) {
  __shared__ uint32_t sh_acc[kProbeWaves];
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int lo = (int)((int64_t)n_tiles * wg / nwg), hi = (int)((int64_t)n_tiles * (wg + 1) / nwg);
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int mine = hi - lo > w ? (hi - lo - w + kProbeWaves - 1) / kProbeWaves : 0;   // this wave's tiles
  // the wave's j-th tile is lo + w + 8j; lane l holds the id of tile 64·round + l
  auto id_of = [&](int j) { return j < mine ? ids[lo + w + kProbeWaves * j] : -1; };
  uint32_t acc = 0;
  int next_ids = id_of(lane);
  for (int base = 0; base < mine; base += kWave) {
    const int my_ids = next_ids;
    next_ids = id_of(base + kWave + lane);
    const int cnt = min(kWave, mine - base);
    for (int j = 0; j < cnt; j += kInFlight) {
      uint4 x[kInFlight][kLoadsPerTile];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int id = __builtin_amdgcn_readlane(my_ids, min(j + u, kWave - 1));
        const bool ok = j + u < cnt && id >= 0 && (int64_t)id < buf_tiles;
        const uint8_t* tile = buf + (size_t)(ok ? id : 0) * kTileBytes;
        const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tile), 0,
                                                         __builtin_amdgcn_readfirstlane(ok ? kTileBytes : 0),
                                                         kBufferRsrcWord3);
#pragma unroll
        for (int k = 0; k < kLoadsPerTile; ++k) x[u][k] = buffer_load16_stream(r, (k * kWave + lane) * 16);
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u)
#pragma unroll
        for (int k = 0; k < kLoadsPerTile; ++k) acc ^= x[u][k].x ^ x[u][k].y ^ x[u][k].z ^ x[u][k].w;
    }
  }
  // fold the workgroup's lanes: XOR over the wave, then over the waves
#pragma unroll
  for (int off = kWave / 2; off > 0; off /= 2) acc ^= (uint32_t)__shfl_xor((int)acc, off, kWave);
  if (lane == 0) sh_acc[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < kProbeWaves; ++i) t ^= sh_acc[i];
    sink[wg] = t;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t buf_tiles, const int32_t* ids, int n_tiles, int num_wgs,
                              uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)num_wgs), dim3(kProbeWaves * kWave), 0, s,
                     static_cast<const uint8_t*>(buf), buf_tiles, ids, n_tiles, sink);
  return hipGetLastError();
}

}  // namespace pkv
