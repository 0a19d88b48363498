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
// One workgroup moves one block of one cache with 16-byte accesses: every load of a
// thread's share is issued before its first store (eight per thread for a 32 KiB block),
// so a block costs one memory round trip.  Loads take the streaming (nontemporal) cache
// policy -- a moved block is not read again by this kernel -- and stores the ordinary
// one.  (Measured on the 2 048-block moves of the 8B-shaped cache: four loads in flight,
// both policies ordinary, 53 us for a copy-on-write; eight in flight 45 us; streaming
// loads 42 us, against 48 us for one contiguous device copy of the same bytes; streaming
// stores as well 58 us.)  An ID outside [0, num_blocks) skips its pair or row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kMoveThreads = 256;
constexpr int kMoveUnroll = 8;  // 16-byte loads in flight per thread

// src / dst: base addresses; a null ID array means "row i of a contiguous buffer".
// Whole rounds of kMoveUnroll pieces per thread use plain global accesses; the last,
// partial round of a block that is not a multiple of kMoveUnroll * kMoveThreads pieces
// goes through buffer resources that cover exactly the source and destination block,
// so its pieces past the block's end load zeros and store nothing, without a branch.
// (Buffer accesses for every round measured 0.6-0.9 us slower on 32 KiB blocks.)
typedef uint32_t move16_t __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(kMoveThreads)
move_blocks_kernel(const uint8_t* k_src, const uint8_t* v_src, const int32_t* src_ids, uint8_t* k_dst,
                   uint8_t* v_dst, const int32_t* dst_ids, int64_t block_bytes, int64_t num_blocks) {
  const int64_t i = blockIdx.x;
  const int64_t s = src_ids ? (int64_t)src_ids[i] : i;
  const int64_t d = dst_ids ? (int64_t)dst_ids[i] : i;
  // IDs address the cache side; buffer rows i < num are always in range
  if (s < 0 || d < 0 || (src_ids && s >= num_blocks) || (dst_ids && d >= num_blocks)) return;
  const uint8_t* from = (blockIdx.y == 0 ? k_src : v_src) + s * block_bytes;
  uint8_t* to = (blockIdx.y == 0 ? k_dst : v_dst) + d * block_bytes;
  const int n = (int)(block_bytes / 16);  // pieces; block_bytes < 2^31, checked by the launcher
  constexpr int U = kMoveUnroll;
  int e = threadIdx.x;
  for (; e + (U - 1) * kMoveThreads < n; e += U * kMoveThreads) {
    move16_t x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = __builtin_nontemporal_load((const move16_t*)from + e + u * kMoveThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) ((move16_t*)to)[e + u * kMoveThreads] = x[u];
  }
  if (e - (int)threadIdx.x >= n) return;  // every piece of this thread came in whole rounds
  const __amdgpu_buffer_rsrc_t rf = tile_rsrc(from, (int)block_bytes);
  const __amdgpu_buffer_rsrc_t rt = tile_rsrc(to, (int)block_bytes);
  u32x4_t x[U];
#pragma unroll
  for (int u = 0; u < U; ++u)
    x[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rf, 16 * (e + u * kMoveThreads), 0, kAuxNT));
#pragma unroll
  for (int u = 0; u < U; ++u) __builtin_amdgcn_raw_buffer_store_b128(x[u], rt, 16 * (e + u * kMoveThreads), 0, 0);
}

hipError_t launch_move_blocks(const void* k_src, const void* v_src, const int32_t* src_ids, void* k_dst,
                              void* v_dst, const int32_t* dst_ids, int32_t num, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream) {
  static_assert(16 * kMoveUnroll * kMoveThreads <= ((int64_t)1 << 31) - kMoveMaxBlockBytes, "round headroom");
  if (block_bytes <= 0 || block_bytes >= kMoveMaxBlockBytes) return hipErrorInvalidValue;
  hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)num, 2), dim3(kMoveThreads), 0, stream,
                     (const uint8_t*)k_src, (const uint8_t*)v_src, src_ids, (uint8_t*)k_dst,
                     (uint8_t*)v_dst, dst_ids, block_bytes, num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
