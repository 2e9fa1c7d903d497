// Measuring aid, not part of the attention path: a read-only stream over a list of
// tiles, to measure the HBM read rate this GPU achieves for a given access pattern
// (contiguous, or the paged decode pattern of scattered 2-8 KiB K/V tiles).  The
// decode kernel's bytes per second are then compared with it as well as with the
// published peak.
//
// Wave w of the W waves in the grid reads a contiguous share of the tile list (the
// indices of 64 tiles per round trip); each tile is read with 16-byte-per-lane loads
// (one KiB per wave instruction), four KiB of loads in flight per wave before any is
// consumed.  Every loaded word is folded into one XOR per wave, stored to sink[w], so
// that no load can be dropped.
#include "pkv_device.h"
#include "pkv_internal.h"
#include "pagedkv_probe.h"

namespace pkv {

__global__ __launch_bounds__(kThreads) void read_probe_kernel(
    const uint4 *__restrict__ base, const int32_t *__restrict__ tiles, int32_t num_tiles,
    int32_t tile_vecs, int64_t base_tiles, uint32_t *__restrict__ sink) {
  constexpr int kUnroll = 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x * kWaves + wave;
  const int W = gridDim.x * kWaves;
  const int per_tile = tile_vecs / 64;  // wave instructions per tile
  const int per_wave = (num_tiles + W - 1) / W;
  const int t_begin = min(num_tiles, w * per_wave);
  const int t_end = min(num_tiles, t_begin + per_wave);
  uint32_t acc = 0;
  for (int c0 = t_begin; c0 < t_end; c0 += 64) {
    const int nc = min(64, t_end - c0);
    // Lane i holds the index of tile c0 + i (one round trip per 64 tiles).
    int my = lane < nc ? tiles[c0 + lane] : 0;
    my = my < 0 ? 0 : (my >= base_tiles ? (int)(base_tiles - 1) : my);
    const int nl = nc * per_tile;  // wave load instructions of this chunk
    for (int l = 0; l < nl; l += kUnroll) {
      uint4 x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int ll = min(l + u, nl - 1);  // past the end: re-read the last piece
        const int k = ll / per_tile;
        const int j = ll - k * per_tile;
        const int64_t idx = readlane(my, k);
        x[u] = base[idx * tile_vecs + (int64_t)j * 64 + lane];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
    }
  }
  acc = __builtin_amdgcn_readfirstlane(acc) ^ (uint32_t)lane;  // keep every lane's loads
  if (lane == 0) sink[w] = acc;
}

}  // namespace pkv

extern "C" pkv_status pkv_read_probe(const void *base, int64_t base_bytes, const int32_t *tiles,
                                     int32_t num_tiles, int32_t tile_bytes, uint32_t *sink,
                                     int32_t grid, void *stream) {
  if (!base || !tiles || !sink || num_tiles < 0 || grid <= 0 || tile_bytes <= 0 ||
      tile_bytes % 1024 != 0 || base_bytes < tile_bytes)
    return PKV_ERR_INVALID_ARG;
  if (num_tiles == 0) return PKV_OK;
  const int64_t base_tiles = base_bytes / tile_bytes;
  pkv::read_probe_kernel<<<dim3(grid), dim3(pkv::kThreads), 0,
                           static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4 *>(base), tiles, num_tiles, tile_bytes / 16, base_tiles, sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}
