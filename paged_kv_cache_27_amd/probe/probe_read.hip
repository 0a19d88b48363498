// Streaming-read probe (measurement only): the decode's K/V tile reads with no
// arithmetic, to measure the achievable read rate of that access pattern.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_probe.h"

namespace {

using pkv::load_kv16;
using pkv::tile_rsrc;

constexpr int kWaves = 8;  // one workgroup of 8 waves per CU, as the balanced decode

// TB: tile bytes (a multiple of 1 KiB: L 16-byte loads per lane for each of K and V).
// DEPTH tiles' loads are issued before any is folded: ~16 KiB in flight per wave.
template <int TB>
__global__ void __launch_bounds__(64 * kWaves)
probe_read_kernel(const uint8_t* kc, const uint8_t* vc, const int32_t* tiles, int64_t n, uint32_t* sink) {
  constexpr int L = TB / 1024;
  constexpr int DEPTH = TB >= 8192 ? 1 : 8192 / TB;
  const int lane = threadIdx.x & 63;
  const int64_t W = (int64_t)gridDim.x * kWaves;
  const int64_t w = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t b = n * w / W, e = n * (w + 1) / W;  // this wave's tiles [b, e)
  uint32_t x = 0;
  if (b >= e) return;
  // tile indices one iteration ahead (clamped to the last tile; scalar loads)
  int32_t nxt[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) nxt[d] = tiles[min(b + d, e - 1)];
  for (int64_t i = b; i < e; i += DEPTH) {
    int32_t cur[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      cur[d] = nxt[d];
      nxt[d] = tiles[min(i + DEPTH + d, e - 1)];
    }
    uint4 r[DEPTH][2 * L];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const bool live = i + d < e;  // past the end: an empty resource, zeros, no access
      const size_t off = (size_t)(uint32_t)cur[d] * TB;
      const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kc + off, live ? TB : 0);
      const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vc + off, live ? TB : 0);
#pragma unroll
      for (int c = 0; c < L; ++c) {
        r[d][c] = load_kv16<true>(kr, 1024 * c + 16 * lane);
        r[d][L + c] = load_kv16<true>(vr, 1024 * c + 16 * lane);
      }
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
#pragma unroll
      for (int c = 0; c < 2 * L; ++c) x ^= r[d][c].x ^ r[d][c].y ^ r[d][c].z ^ r[d][c].w;
  }
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace

extern "C" int pkv_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles,
                                    int64_t num_tiles, int32_t tile_bytes, uint32_t* sink, hipStream_t stream) {
  if (num_tiles < 0) return -3;
  if (num_tiles == 0) return 0;
  if (!k_cache || !v_cache || !tiles || !sink) return -1;
  if (((uintptr_t)k_cache & 15) || ((uintptr_t)v_cache & 15)) return -3;
  if (tile_bytes != 1024 && tile_bytes != 2048 && tile_bytes != 4096 && tile_bytes != 8192) return -3;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -6;
  const uint8_t* kc = (const uint8_t*)k_cache;
  const uint8_t* vc = (const uint8_t*)v_cache;
  const dim3 grid(cus), block(64 * kWaves);
  switch (tile_bytes) {
    case 1024: hipLaunchKernelGGL(probe_read_kernel<1024>, grid, block, 0, stream, kc, vc, tiles, num_tiles, sink); break;
    case 2048: hipLaunchKernelGGL(probe_read_kernel<2048>, grid, block, 0, stream, kc, vc, tiles, num_tiles, sink); break;
    case 4096: hipLaunchKernelGGL(probe_read_kernel<4096>, grid, block, 0, stream, kc, vc, tiles, num_tiles, sink); break;
    case 8192: hipLaunchKernelGGL(probe_read_kernel<8192>, grid, block, 0, stream, kc, vc, tiles, num_tiles, sink); break;
    default: return -3;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
