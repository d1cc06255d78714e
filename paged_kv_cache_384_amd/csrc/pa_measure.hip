// The bandwidth reference of the decode access pattern (measurement only): whole tiles of two
// pools read in a given order with the attention kernel's loads, so that the attention kernel's
// rate can be set beside what plain reads of the same bytes, in the same pattern, reach.
//
// Source (page title, section): "PagedAttention 심층 분석 — LLM KV 캐시 메모리 관리"
// (ryotta.opik.net), §2 and §5: blocks sit wherever the pool had room, and decode attention is
// bound by reading them; the reference therefore reads tiles in a random order, not in sequence.
#include "pa_device.h"

namespace pa {

// Wavefront w reads tiles [w * kMeasureTilesPerWave, +kMeasureTilesPerWave) of the order: for
// each, tile_bytes / 1024 non-temporal 16-byte wave loads of 1 KiB from each pool (lane l at
// byte 16 l of each KiB), and folds every word with XOR; the wave's fold goes to sink[w].
__global__ __launch_bounds__(256) void tile_read_kernel(MeasureArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t first = wave * kMeasureTilesPerWave;
  if (first >= a.num_tiles) return;
  const int64_t last = first + kMeasureTilesPerWave < a.num_tiles ? first + kMeasureTilesPerWave
                                                                  : a.num_tiles;
  const int kib = a.tile_bytes / 1024;
  uint32_t x = 0;
  for (int64_t t = first; t < last; ++t) {
    const int64_t base = static_cast<int64_t>(a.tiles[t]) * a.tile_bytes + 16 * lane;
    for (int c = 0; c < kib; ++c) {
      const u32x4 p = load16_kv<true>(a.pool_a + base + c * 1024);
      const u32x4 q = load16_kv<true>(a.pool_b + base + c * 1024);
      x ^= p.x ^ p.y ^ p.z ^ p.w ^ q.x ^ q.y ^ q.z ^ q.w;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, 64));
  if (lane == 0) a.sink[wave] = x;
}

hipError_t launch_tile_read(const MeasureArgs& a, hipStream_t stream) {
  if (a.num_tiles == 0) return hipSuccess;
  const int64_t waves = (a.num_tiles + kMeasureTilesPerWave - 1) / kMeasureTilesPerWave;
  hipLaunchKernelGGL(tile_read_kernel, dim3(static_cast<unsigned>((waves + 3) / 4)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace pa
