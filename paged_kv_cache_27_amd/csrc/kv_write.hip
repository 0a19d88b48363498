// Slot resolution and the scatter-write of new K/V into the paged cache.
//
// Slot resolution follows the block-table lookup of "Optimizacion de Inferencia
// LLM", section "PagedAttention: Conceptos de SO..." (get_physical_block: entry
// position / B, offset position % B).  The write stores each new token's K and V
// at (block, offset) of every KV head ("PagedAttention por dentro...", section
// "La tabla de paginas (block table)").
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

// Slot of token t: block_tables[seq][pos / B] * B + pos % B, or -1 for a negative
// position or sequence ID or a position past the table's row.
__device__ __forceinline__ int64_t resolve_slot(const int32_t* __restrict__ seq_ids,
                                                const int32_t* __restrict__ positions, int64_t t,
                                                const int32_t* __restrict__ block_tables,
                                                int32_t max_blocks_per_seq, int32_t block_size) {
  const int32_t pos = positions[t], seq = seq_ids[t];
  if (pos < 0 || seq < 0 || pos / block_size >= max_blocks_per_seq) return -1;
  const int64_t entry = (int64_t)seq * max_blocks_per_seq + pos / block_size;
  return (int64_t)block_tables[entry] * block_size + pos % block_size;
}

__global__ void __launch_bounds__(256)
slot_mapping_kernel(const int32_t* __restrict__ seq_ids, const int32_t* __restrict__ positions,
                    int32_t num_tokens, const int32_t* __restrict__ block_tables,
                    int32_t max_blocks_per_seq, int32_t block_size,
                    int64_t* __restrict__ slot_mapping) {
  const int32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  slot_mapping[t] = resolve_slot(seq_ids, positions, t, block_tables, max_blocks_per_seq, block_size);
}

// Where each token goes: the given slots, or (RESOLVE) slots resolved here from
// sequence IDs, positions and block tables -- the slot resolution and the write in one
// launch -- and stored to slot_out when it is not null.
struct SlotSrc {
  const int64_t* slot_mapping;
  const int32_t* seq_ids;
  const int32_t* positions;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  int64_t* slot_out;
};

// One work item = 8 consecutive elements of one (token, KV head) row, for K and V.
template <int SRC, int DST, bool RESOLVE>
__global__ void __launch_bounds__(256)
kv_write_kernel(const SlotSrc ss, int32_t num_tokens,
                const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
                uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_slots,
                float k_scale, float v_scale) {
  constexpr int SB = DtInfo<SRC>::bytes;
  constexpr int DB = DtInfo<DST>::bytes;
  const int32_t per_row = head_dim / 8;
  const int64_t items = (int64_t)num_tokens * num_kv_heads * per_row;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items;
       it += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = it / per_row;  // token * H + head
    const int32_t d0 = (int32_t)(it - row * per_row) * 8;
    const int64_t t = row / num_kv_heads;
    const int32_t h = (int32_t)(row - t * num_kv_heads);
    int64_t slot;
    if constexpr (RESOLVE) {
      slot = resolve_slot(ss.seq_ids, ss.positions, t, ss.block_tables, ss.max_blocks_per_seq, block_size);
      if (ss.slot_out && h == 0 && d0 == 0) ss.slot_out[t] = slot;
    } else {
      slot = ss.slot_mapping[t];
    }
    if (slot < 0 || slot >= num_slots) continue;  // no slot, or none of this cache's
    const int64_t blk = slot / block_size;
    const int32_t off = (int32_t)(slot - blk * block_size);
    const int64_t src = (row * head_dim + d0) * SB;
    const int64_t dst = (((blk * num_kv_heads + h) * block_size + off) * head_dim + d0) * DB;
    if constexpr (SRC == DST) {
      // bit copy: 8 elements = 8 * SB bytes (16 or 32)
#pragma unroll
      for (int b = 0; b < SB / 2; ++b) {
        *(uint4*)(k_cache + dst + 16 * b) = *(const uint4*)(k + src + 16 * b);
        *(uint4*)(v_cache + dst + 16 * b) = *(const uint4*)(v + src + 16 * b);
      }
    } else {
      static_assert(DST == kFP8, "only a bit copy or an fp8 quantisation is supported");
      constexpr int W = Unpack8<SRC>::words;
      uint32_t kw[W], vw[W];
#pragma unroll
      for (int i = 0; i < W; ++i) {
        kw[i] = *(const uint32_t*)(k + src + 4 * i);
        vw[i] = *(const uint32_t*)(v + src + 4 * i);
      }
      float kf[8], vf[8];
      Unpack8<SRC>::run(kw, kf);
      Unpack8<SRC>::run(vw, vf);
      uint32_t ko[2] = {0, 0}, vo[2] = {0, 0};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // IEEE division (correctly rounded), as the stored code is defined on x / scale.
        ko[i / 4] |= f32_to_e4m3_satfinite(kf[i] / k_scale) << (8 * (i % 4));
        vo[i / 4] |= f32_to_e4m3_satfinite(vf[i] / v_scale) << (8 * (i % 4));
      }
      *(uint2*)(k_cache + dst) = make_uint2(ko[0], ko[1]);
      *(uint2*)(v_cache + dst) = make_uint2(vo[0], vo[1]);
    }
  }
}

hipError_t launch_slot_mapping(const int32_t* seq_ids, const int32_t* positions, int32_t n,
                               const int32_t* block_tables, int32_t max_blocks,
                               int32_t block_size, int64_t* slots, hipStream_t stream) {
  const int threads = 256;
  const int blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), 0, stream, seq_ids,
                     positions, n, block_tables, max_blocks, block_size, slots);
  return hipGetLastError();
}

template <int SRC, int DST>
static hipError_t launch_write_t(const WriteArgs& a, hipStream_t stream) {
  const int threads = 256;
  const int64_t items = (int64_t)a.num_tokens * a.num_kv_heads * (a.head_dim / 8);
  int64_t blocks = (items + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  const SlotSrc ss{a.slot_mapping, a.seq_ids, a.positions, a.block_tables, a.max_blocks_per_seq, a.slot_out};
  if (a.seq_ids)
    hipLaunchKernelGGL((kv_write_kernel<SRC, DST, true>), dim3((unsigned)blocks), dim3(threads), 0,
                       stream, ss, a.num_tokens, (const uint8_t*)a.k, (const uint8_t*)a.v,
                       (uint8_t*)a.k_cache, (uint8_t*)a.v_cache, a.num_kv_heads, a.head_dim,
                       a.block_size, a.num_blocks * a.block_size, a.k_scale, a.v_scale);
  else
    hipLaunchKernelGGL((kv_write_kernel<SRC, DST, false>), dim3((unsigned)blocks), dim3(threads), 0,
                       stream, ss, a.num_tokens, (const uint8_t*)a.k, (const uint8_t*)a.v,
                       (uint8_t*)a.k_cache, (uint8_t*)a.v_cache, a.num_kv_heads, a.head_dim,
                       a.block_size, a.num_blocks * a.block_size, a.k_scale, a.v_scale);
  return hipGetLastError();
}

hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream) {
  if (a.src_dtype == a.cache_dtype) {
    switch (a.src_dtype) {
      case kF32: return launch_write_t<kF32, kF32>(a, stream);
      case kF16: return launch_write_t<kF16, kF16>(a, stream);
      case kBF16: return launch_write_t<kBF16, kBF16>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (a.cache_dtype == kFP8) {
    switch (a.src_dtype) {
      case kF32: return launch_write_t<kF32, kFP8>(a, stream);
      case kF16: return launch_write_t<kF16, kFP8>(a, stream);
      case kBF16: return launch_write_t<kBF16, kFP8>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
