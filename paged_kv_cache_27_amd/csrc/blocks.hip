// Whole-block moves of the paged cache for gfx950: copy-on-write copies and swap
// out / in.
//
// A physical block of one layer's cache is H_kv * B * d_h elements, contiguous (the
// cache layout is [num_blocks][H_kv][B][d_h]).  Every move below copies whole blocks of
// the K cache and of the V cache:
//   * copy-on-write: block src[i] -> block dst[i] ("PagedAttention por dentro...",
//     section "Copy-on-write para sampling paralelo"; "La despensa por casilleros",
//     section "Prefix caching...": a shared block is copied for the branch about to
//     write into it, and only then written);
//   * swap out: block ids[i] -> row i of a contiguous buffer, swap in: the reverse
//     (same page, section "Estrategia 2: swap": an evicted session's blocks go to CPU
//     RAM and come back when it resumes).  The buffer may be device memory or pinned
//     host memory (then the kernel's stores and loads cross PCIe).
// One workgroup moves one block of one cache with 16-byte accesses, four in flight per
// thread.  An ID outside [0, num_blocks) skips its pair or row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {

constexpr int kMoveThreads = 256;

// src / dst: base addresses; a null ID array means "row i of a contiguous buffer".
__global__ void __launch_bounds__(kMoveThreads)
move_blocks_kernel(const uint8_t* k_src, const uint8_t* v_src, const int32_t* src_ids, uint8_t* k_dst,
                   uint8_t* v_dst, const int32_t* dst_ids, int64_t block_bytes, int64_t num_blocks) {
  const int64_t i = blockIdx.x;
  const int64_t s = src_ids ? (int64_t)src_ids[i] : i;
  const int64_t d = dst_ids ? (int64_t)dst_ids[i] : i;
  // IDs address the cache side; buffer rows i < num are always in range
  if (s < 0 || d < 0 || (src_ids && s >= num_blocks) || (dst_ids && d >= num_blocks)) return;
  const uint4* from = (const uint4*)((blockIdx.y == 0 ? k_src : v_src) + s * block_bytes);
  uint4* to = (uint4*)((blockIdx.y == 0 ? k_dst : v_dst) + d * block_bytes);
  const int64_t n = block_bytes / 16;
  constexpr int U = 4;
  int64_t e = threadIdx.x;
  for (; e + (U - 1) * kMoveThreads < n; e += U * kMoveThreads) {
    uint4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = from[e + u * kMoveThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) to[e + u * kMoveThreads] = x[u];
  }
  for (; e < n; e += kMoveThreads) to[e] = from[e];
}

hipError_t launch_move_blocks(const void* k_src, const void* v_src, const int32_t* src_ids, void* k_dst,
                              void* v_dst, const int32_t* dst_ids, int32_t num, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream) {
  hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)num, 2), dim3(kMoveThreads), 0, stream,
                     (const uint8_t*)k_src, (const uint8_t*)v_src, src_ids, (uint8_t*)k_dst,
                     (uint8_t*)v_dst, dst_ids, block_bytes, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
