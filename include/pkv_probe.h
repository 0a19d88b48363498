/* Streaming-read probe: a measurement kernel, not part of the attention path.
 *
 * It reads the K and V tiles of a list -- each tile one 16-token row range of one
 * (physical block, KV head) of the paged caches, listed in the order a decode visits
 * them -- with the decode kernel's load shape (16-byte nontemporal buffer loads, one
 * workgroup of 8 waves per CU, the list split evenly over the waves, about 16 KiB of
 * loads in flight per wave) and only XOR-folds what it loads.  Its rate is the
 * achievable read rate of that access pattern on this device: the ceiling the
 * decode's streaming is compared with.
 *
 * Callers: measurement scripts (the benchmark), which allocate everything.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 *   k_cache, v_cache : device pointers to the caches (16-byte aligned)
 *   tiles            : int32 [num_tiles] device; tile t covers bytes
 *                      [tiles[t] * tile_bytes, (tiles[t] + 1) * tile_bytes) of each cache
 *                      (every index must lie inside both caches: unchecked)
 *   tile_bytes       : 16 * head_dim * element bytes: 1024, 2048, 4096 or 8192
 *   sink             : device pointer to 4 writable bytes (written only if the fold of
 *                      everything read hits one fixed value, so that no load is elided)
 * Asynchronous on `stream`; allocates nothing.  Returns 0, -1 for a null pointer, -3 for
 * an unsupported tile size, a negative count or misaligned caches, -6 for a launch error.
 */
int pkv_probe_read_tiles(const void* k_cache, const void* v_cache, const int32_t* tiles, int64_t num_tiles,
                         int32_t tile_bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
