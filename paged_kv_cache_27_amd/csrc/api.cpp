// C ABI layer: host-side argument checks, partition choice, workspace carving and
// dispatch to the gfx950 kernels.  Declarations and contracts: include/pagedkv.h.
#include "pagedkv.h"

#include <hip/hip_runtime.h>

#include "pkv_launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool known_dtype(int d) { return d >= PKV_F32 && d <= PKV_FP8_E4M3; }

int check_cache(const pkv_cache_desc* c) {
  if (!c) return PKV_ERR_NULL;
  if (!known_dtype(c->dtype)) return PKV_ERR_DTYPE;
  if (c->block_size != 16 && c->block_size != 32) return PKV_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_SHAPE;
  if (c->num_kv_heads <= 0 || c->num_blocks <= 0) return PKV_ERR_SHAPE;
  if (c->dtype == PKV_FP8_E4M3 && !(c->k_scale > 0.0f && c->v_scale > 0.0f)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Tokens per partition for partition_size == 0.  Each (sequence, KV head) with a
// context longer than 512 tokens is cut into 512-token partitions: enough
// workgroups to fill 256 compute units even for a handful of sequences, and a
// partial-result overhead (G * (d_h + 2) floats per partition) under 1% of the
// K/V bytes a partition reads.
int32_t auto_partition(int32_t max_context_len, int32_t block_size) {
  const int32_t p = 512;
  if (max_context_len <= p) return 0;
  return (p / block_size) * block_size;
}

struct Plan {
  int32_t partition;
  int32_t parts;
};

int plan_partitions(int32_t requested, int32_t max_context_len, int32_t block_size, Plan* out) {
  int32_t p;
  if (requested == -1) {
    p = 0;
  } else if (requested == 0) {
    p = auto_partition(max_context_len, block_size);
  } else {
    if (requested < 0 || requested % block_size != 0) return PKV_ERR_WORKSPACE;
    p = requested;
  }
  if (p == 0 || max_context_len <= p) {
    // single pass: one partition spanning the longest context
    int32_t span = max_context_len > 0 ? max_context_len : block_size;
    span = (span + block_size - 1) / block_size * block_size;
    out->partition = span;
    out->parts = 1;
  } else {
    out->partition = p;
    out->parts = (max_context_len + p - 1) / p;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return 1; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case PKV_ERR_SHAPE: return "unsupported head_dim / block_size / group size, or bad sizes";
    case PKV_ERR_HEADS: return "num_q_heads is not a multiple of num_kv_heads";
    case PKV_ERR_WORKSPACE: return "workspace too small or bad partition size";
    case PKV_ERR_LAUNCH: return "HIP launch error";
    default: return "unknown status";
  }
}

int paged_kv_slot_mapping(const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t block_size, int64_t* slot_mapping, hipStream_t stream) {
  if (num_tokens < 0 || block_size <= 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!seq_ids || !positions || !block_tables || !slot_mapping) return PKV_ERR_NULL;
  hipError_t e = pkv::launch_slot_mapping(seq_ids, positions, num_tokens, block_tables,
                                          max_blocks_per_seq, block_size, slot_mapping, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_write(const int64_t* slot_mapping, int32_t num_tokens, const void* k,
                   const void* v, pkv_dtype src_dtype, void* k_cache, void* v_cache,
                   const pkv_cache_desc* cache, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (!known_dtype(src_dtype) || src_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (cache->dtype != src_dtype && cache->dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (num_tokens == 0) return PKV_OK;
  if (!slot_mapping || !k || !v || !k_cache || !v_cache) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_SHAPE;
  pkv::WriteArgs a;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.k = k;
  a.v = v;
  a.src_dtype = src_dtype;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.cache_dtype = cache->dtype;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.block_size = cache->block_size;
  a.k_scale = cache->dtype == PKV_FP8_E4M3 ? cache->k_scale : 1.0f;
  a.v_scale = cache->dtype == PKV_FP8_E4M3 ? cache->v_scale : 1.0f;
  hipError_t e = pkv::launch_kv_write(a, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t paged_attention_auto_partition(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t block_size) {
  (void)num_seqs;
  (void)num_kv_heads;
  if (block_size <= 0) return 0;
  return auto_partition(max_context_len, block_size);
}

size_t paged_attention_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_context_len, int32_t block_size,
                                      int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || block_size <= 0) return 0;
  Plan plan;
  if (plan_partitions(partition_size, max_context_len, block_size, &plan)) return 0;
  if (plan.parts <= 1) return 0;
  return pkv::ws_total_bytes(num_seqs, num_q_heads, head_dim, plan.parts);
}

int paged_attention_decode(const void* q, pkv_dtype q_dtype, int32_t num_seqs,
                           int32_t num_q_heads, const void* k_cache, const void* v_cache,
                           const pkv_cache_desc* cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, float scale, void* out,
                           pkv_dtype out_dtype, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (!known_dtype(q_dtype) || !known_dtype(out_dtype)) return PKV_ERR_DTYPE;
  if (q_dtype == PKV_FP8_E4M3 || out_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (cache->dtype == PKV_FP8_E4M3) {
    if (q_dtype != PKV_BF16 && q_dtype != PKV_F16) return PKV_ERR_DTYPE;
  } else if (cache->dtype != q_dtype) {
    return PKV_ERR_DTYPE;
  }
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || max_blocks_per_seq <= 0)
    return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || cache->num_kv_heads > 65535) return PKV_ERR_SHAPE;
  if (num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_HEADS;
  const int32_t G = num_q_heads / cache->num_kv_heads;
  if (G < 1 || G > 16) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size < max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_SHAPE;

  Plan plan;
  st = plan_partitions(partition_size, max_context_len, cache->block_size, &plan);
  if (st) return st;

  pkv::DecodeArgs a;
  a.q = q;
  a.q_dtype = q_dtype;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.head_dim = cache->head_dim;
  a.block_size = cache->block_size;
  a.cache_dtype = cache->dtype;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.out = out;
  a.out_dtype = out_dtype;
  a.partition = plan.partition;
  a.num_partitions = plan.parts;
  a.ws_m = a.ws_l = a.ws_acc = nullptr;
  if (plan.parts > 1) {
    const size_t need = pkv::ws_total_bytes(num_seqs, num_q_heads, cache->head_dim, plan.parts);
    if (!workspace) return PKV_ERR_NULL;
    if (workspace_bytes < need || ((uintptr_t)workspace & 255u)) return PKV_ERR_WORKSPACE;
    const size_t ml = pkv::ws_ml_bytes(num_seqs, num_q_heads, plan.parts);
    a.ws_m = (float*)workspace;
    a.ws_l = (float*)((char*)workspace + ml);
    a.ws_acc = (float*)((char*)workspace + 2 * ml);
  }
  hipError_t e = pkv::launch_decode(a, stream);
  if (e == hipErrorInvalidValue) return PKV_ERR_SHAPE;
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
