// C ABI layer: host-side argument checks, schedule choice, workspace carving and
// dispatch to the gfx950 kernels.  Declarations and contracts: include/pagedkv.h.
#include "pagedkv.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "pkv_launch.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool known_dtype(int d) { return d >= PKV_F32 && d <= PKV_FP8_E4M3; }

// Streaming K/V loads unless the caller says blocks are shared between sequences.
bool kv_stream(const pkv_cache_desc* c) { return (c->flags & PKV_CACHE_SHARED_BLOCKS) == 0; }

int check_cache(const pkv_cache_desc* c) {
  if (!c) return PKV_ERR_NULL;
  if (!known_dtype(c->dtype)) return PKV_ERR_DTYPE;
  if (c->block_size != 16 && c->block_size != 32) return PKV_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_SHAPE;
  if (c->num_kv_heads <= 0 || c->num_blocks <= 0) return PKV_ERR_SHAPE;
  if (c->dtype == PKV_FP8_E4M3 && !(c->k_scale > 0.0f && c->v_scale > 0.0f)) return PKV_ERR_SHAPE;
  if (c->flags & ~PKV_CACHE_SHARED_BLOCKS) return PKV_ERR_SHAPE;
  return PKV_OK;
}

int check_decode_shape(const pkv_cache_desc* cache, int q_dtype, int out_dtype, int32_t num_seqs,
                       int32_t num_q_heads, int32_t max_context_len) {
  int st = check_cache(cache);
  if (st) return st;
  if (!known_dtype(q_dtype) || !known_dtype(out_dtype)) return PKV_ERR_DTYPE;
  if (q_dtype == PKV_FP8_E4M3 || out_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (cache->dtype == PKV_FP8_E4M3) {
    if (q_dtype != PKV_BF16 && q_dtype != PKV_F16) return PKV_ERR_DTYPE;
  } else if (cache->dtype != q_dtype) {
    return PKV_ERR_DTYPE;
  }
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0) return PKV_ERR_SHAPE;
  if (num_seqs > 65535 || cache->num_kv_heads > 65535) return PKV_ERR_SHAPE;
  if (num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_HEADS;
  const int32_t G = num_q_heads / cache->num_kv_heads;
  if (G < 1 || G > 16) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Bytes of one physical block of one cache: H_kv * B * d_h elements.
int64_t block_bytes(const pkv_cache_desc* c) {
  const int64_t eb = c->dtype == PKV_F32 ? 4 : (c->dtype == PKV_FP8_E4M3 ? 1 : 2);
  return (int64_t)c->num_kv_heads * c->block_size * c->head_dim * eb;
}

// How a decode call is scheduled.
enum Mode { kSingle = 0, kFixed = 1, kBalanced = 2 };

struct Plan {
  Mode mode;
  int32_t partition;  // tokens per partition (fixed / single)
  int32_t parts;      // partitions in the grid (fixed / single)
  int32_t workers;    // waves in the launch (balanced)
  size_t ws_bytes;
};

// partition_size == 0 picks the balanced schedule (up to kStreamKMaxSeqs sequences;
// beyond that, fixed 512-token partitions); -1 one pass per (sequence, KV head);
// > 0 fixed partitions of that many tokens (a multiple of the block size).
int plan_decode(const pkv_cache_desc* c, int q_dtype, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_context_len, int32_t requested, Plan* out) {
  const int32_t bs = c->block_size;
  const int32_t G = num_q_heads / c->num_kv_heads;
  pkv::SkPlan sk;
  if (requested == 0 && num_seqs <= pkv::kStreamKMaxSeqs &&
      pkv::streamk_plan(c->dtype, q_dtype, c->head_dim, G, num_seqs, kv_stream(c), false, &sk) == 0) {
    out->mode = kBalanced;
    out->partition = 0;
    out->parts = 0;
    out->workers = sk.waves;
    out->ws_bytes = sk.ws_bytes;
    return PKV_OK;
  }
  int32_t p;
  if (requested == -1) {
    p = 0;
  } else if (requested == 0) {
    p = (512 / bs) * bs;
  } else {
    if (requested < 0 || requested % bs != 0) return PKV_ERR_WORKSPACE;
    p = requested;
  }
  out->workers = 0;
  if (p == 0 || max_context_len <= p) {
    // one pass: a single partition spanning the longest context
    int32_t span = max_context_len > 0 ? max_context_len : bs;
    span = (span + bs - 1) / bs * bs;
    out->mode = kSingle;
    out->partition = span;
    out->parts = 1;
    out->ws_bytes = 0;
  } else {
    out->mode = kFixed;
    out->partition = p;
    out->parts = (max_context_len + p - 1) / p;
    out->ws_bytes = pkv::ws_total_bytes(num_seqs, num_q_heads, c->head_dim, out->parts);
  }
  return PKV_OK;
}

// The shared-prefix decode: prefix partials, then the balanced suffix pass.
struct PrefixPlan {
  int32_t splits;       // slices of each prefix's chunks (prefix kernel workgroups per row tile)
  int32_t tiles;        // kPrefixRows-row tiles per group
  size_t part_bytes;    // prefix partials
  pkv::SkPlan sk;       // suffix pass
  size_t ws_bytes;
};

int plan_prefix(const pkv_cache_desc* c, int q_dtype, int32_t num_seqs, int32_t num_q_heads,
                int32_t max_context_len, int32_t num_groups, int32_t max_group_size,
                int32_t max_prefix_len, PrefixPlan* out) {
  if (c->dtype == PKV_F32) return PKV_ERR_DTYPE;  // 16-bit and fp8 caches (queries checked as decode)
  if (num_groups < 1 || max_group_size < 1 || max_prefix_len < 0) return PKV_ERR_SHAPE;
  if (max_prefix_len % c->block_size != 0 || max_prefix_len > max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs > pkv::kStreamKMaxSeqs || num_groups > num_seqs) return PKV_ERR_SHAPE;
  const int32_t G = num_q_heads / c->num_kv_heads;
  if (pkv::streamk_plan(c->dtype, q_dtype, c->head_dim, G, num_seqs, true, true, &out->sk) != 0)
    return PKV_ERR_SHAPE;
  out->tiles = (int32_t)(((int64_t)max_group_size * G + pkv::kPrefixRows - 1) / pkv::kPrefixRows);
  // Enough prefix workgroups (4 waves each) for two per CU (the suffix pass runs one
  // workgroup of sk.waves / CUs = 8 waves per CU), at most 8 slices and at most one per
  // 16-token chunk of the longest prefix.  (Every slice adds a partial per row that the
  // suffix pass folds in: on the 256-sequence workload 4 slices measured faster than 8
  // and than 2.)
  const int64_t per_split = (int64_t)num_groups * out->tiles * c->num_kv_heads;
  const int64_t wgs = out->sk.waves / 4 > 0 ? out->sk.waves / 4 : 1;
  int64_t splits = (wgs + per_split - 1) / per_split;
  const int64_t max_splits = max_prefix_len / 16 > 0 ? max_prefix_len / 16 : 1;
  splits = splits < 1 ? 1 : (splits > 8 ? 8 : splits);
  splits = splits > max_splits ? max_splits : splits;
  if (per_split * splits > 0x7fffffff) return PKV_ERR_SHAPE;
  out->splits = (int32_t)splits;
  out->part_bytes = pkv::align256((size_t)num_seqs * num_q_heads * splits * (4 + c->head_dim) * sizeof(float));
  out->ws_bytes = out->sk.ws_bytes + out->part_bytes;
  return PKV_OK;
}

// Checks shared by the two write entry points (num_tokens == 0 returns PKV_OK before
// the pointers are looked at).
int check_write(int32_t num_tokens, const void* k, const void* v, int src_dtype, const void* k_cache,
                const void* v_cache, const pkv_cache_desc* cache) {
  int st = check_cache(cache);
  if (st) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (!known_dtype(src_dtype) || src_dtype == PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (cache->dtype != src_dtype && cache->dtype != PKV_FP8_E4M3) return PKV_ERR_DTYPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// The address a kernel uses for a swap buffer: device memory as it is; pinned host
// memory (hipHostMalloc, which maps it into every GPU's address space) through the
// device address the runtime mapped for it.  Anything else -- pageable host memory, an
// address the runtime does not know -- is refused (non-zero), since a kernel touching it
// would fault.
int device_view(void* p, void** out) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  if (at.type == hipMemoryTypeHost) {
    if (!at.devicePointer) return -1;
    *out = at.devicePointer;
    return 0;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged || at.type == hipMemoryTypeUnified) {
    *out = p;
    return 0;
  }
  return -1;
}

// Write arguments without a slot source (the caller sets one).
pkv::WriteArgs write_args(int32_t num_tokens, const void* k, const void* v, int src_dtype, void* k_cache,
                          void* v_cache, const pkv_cache_desc* cache) {
  pkv::WriteArgs a;
  a.slot_mapping = nullptr;
  a.seq_ids = nullptr;
  a.positions = nullptr;
  a.block_tables = nullptr;
  a.max_blocks_per_seq = 0;
  a.slot_out = nullptr;
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
  a.num_blocks = cache->num_blocks;
  a.k_scale = cache->dtype == PKV_FP8_E4M3 ? cache->k_scale : 1.0f;
  a.v_scale = cache->dtype == PKV_FP8_E4M3 ? cache->v_scale : 1.0f;
  return a;
}

// Arguments common to both uses of the rows kernel; the use-specific ones stay null.
pkv::RowsArgs rows_args(const void* q, int q_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                        const void* v_cache, const pkv_cache_desc* c, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, float scale, int32_t tiles, hipStream_t stream) {
  pkv::RowsArgs p;
  p.q = q;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = c->num_kv_heads;
  p.head_dim = c->head_dim;
  p.block_size = c->block_size;
  p.cache_dtype = c->dtype;
  p.q_dtype = q_dtype;
  p.k_scale = c->dtype == PKV_FP8_E4M3 ? c->k_scale : 1.0f;
  p.v_scale = c->dtype == PKV_FP8_E4M3 ? c->v_scale : 1.0f;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.scale = scale;
  p.tiles = tiles;
  p.stream = stream;
  p.group_starts = nullptr;
  p.prefix_lens = nullptr;
  p.pre_part = nullptr;
  p.splits = 1;
  p.cu_q = nullptr;
  p.context_lens = nullptr;
  p.out = nullptr;
  p.out_dtype = 0;
  return p;
}


// Checks of a decode call's arguments shared by the decode entry points (everything but
// the workspace).
int check_decode_call(const void* q, int q_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
                      const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                      int32_t window, int32_t sinks, const void* out, int out_dtype) {
  int st = check_decode_shape(cache, q_dtype, out_dtype, num_seqs, num_q_heads, max_context_len);
  if (st) return st;
  if (window < 0 || sinks < 0) return PKV_ERR_SHAPE;
  if (max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size < max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Launch a checked and planned decode; `workspace` holds plan.ws_bytes (unused when 0).
int run_decode(const Plan& plan, const void* q, int q_dtype, int32_t num_seqs, int32_t num_q_heads,
               const void* k_cache, const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
               int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, int32_t window,
               int32_t sinks, float scale, void* out, int out_dtype, void* workspace, hipStream_t stream) {
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
  a.kv_stream = kv_stream(cache) ? 1 : 0;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.window = window;
  a.sinks = window > 0 ? sinks : 0;
  a.out = out;
  a.out_dtype = out_dtype;
  a.partition = plan.partition;
  a.num_partitions = plan.parts;
  a.ws_m = a.ws_l = a.ws_acc = nullptr;
  a.sk_workers = plan.workers;
  a.sk_count = nullptr;
  a.sk_part = nullptr;
  a.seq_begin = nullptr;
  a.pre_part = nullptr;
  a.pre_splits = 0;
  char* body = (char*)workspace + pkv::kWsHeaderBytes;  // only used when ws_bytes > 0
  if (plan.mode == kFixed) {
    const size_t ml = pkv::ws_ml_bytes(num_seqs, num_q_heads, plan.parts);
    a.ws_m = (float*)body;
    a.ws_l = (float*)(body + ml);
    a.ws_acc = (float*)(body + 2 * ml);
  } else if (plan.mode == kBalanced) {
    a.sk_count = (int32_t*)workspace;
    a.sk_part = (float*)body;
  }
  hipError_t e = plan.mode == kBalanced ? pkv::launch_decode_streamk(a, stream)
                                        : pkv::launch_decode(a, stream);
  if (e == hipErrorInvalidValue) return PKV_ERR_SHAPE;
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// ---- scratch of the no-alloc decode ------------------------------------------------
// One array per GPU, held from the library's first use on that GPU until the process
// ends.  Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the device address comes from hipGetSymbolAddress,
// once per device with that device current, and is kept per device.
__device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address; on its first use the counter header is cleared
// on `stream` (a fill kernel), and every decode leaves it zero after that.  A first use
// under stream capture only records the fill into the graph (it runs at each replay,
// before the decode recorded after it), so the device is not marked cleared until a
// call outside capture has launched the fill itself.
int scratch_for_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    (void)hipGetLastError();
    return PKV_ERR_LAUNCH;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) {
    *out = ptr;
    return PKV_OK;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) {
      (void)hipGetLastError();
      return PKV_ERR_LAUNCH;
    }
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return PKV_ERR_LAUNCH;
    }
    constexpr int kWords = (int)(pkv::kWsHeaderBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(zero_words_kernel, dim3(kWords / 256), dim3(256), 0, stream, (uint32_t*)ptr, kWords);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_LAUNCH;
    if (capture == hipStreamCaptureStatusNone) g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return PKV_OK;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return 9; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case PKV_ERR_SHAPE: return "unsupported head_dim / block_size / group size, or bad sizes";
    case PKV_ERR_HEADS: return "num_q_heads is not a multiple of num_kv_heads";
    case PKV_ERR_WORKSPACE: return "workspace too small or bad partition size";
    case PKV_ERR_LAUNCH: return "HIP launch error";
    case PKV_ERR_POOL_EXHAUSTED: return "block pool: not enough free blocks";
    case PKV_ERR_BLOCK_STATE: return "block pool: block ID out of range or not allocated";
    case PKV_ERR_SCRATCH: return "the call needs more scratch than the no-alloc decode holds";
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
  int st = check_write(num_tokens, k, v, src_dtype, k_cache, v_cache, cache);
  if (st || num_tokens == 0) return st;
  if (!slot_mapping) return PKV_ERR_NULL;
  pkv::WriteArgs a = write_args(num_tokens, k, v, src_dtype, k_cache, v_cache, cache);
  a.slot_mapping = slot_mapping;
  hipError_t e = pkv::launch_kv_write(a, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_write_positions(const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                             const int32_t* block_tables, int32_t max_blocks_per_seq, const void* k,
                             const void* v, pkv_dtype src_dtype, void* k_cache, void* v_cache,
                             const pkv_cache_desc* cache, int64_t* slot_mapping, hipStream_t stream) {
  int st = check_write(num_tokens, k, v, src_dtype, k_cache, v_cache, cache);
  if (st) return st;
  if (max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!seq_ids || !positions || !block_tables) return PKV_ERR_NULL;
  pkv::WriteArgs a = write_args(num_tokens, k, v, src_dtype, k_cache, v_cache, cache);
  a.seq_ids = seq_ids;
  a.positions = positions;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.slot_out = slot_mapping;
  hipError_t e = pkv::launch_kv_write(a, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_copy_blocks(const int32_t* src_ids, const int32_t* dst_ids, int32_t num_pairs,
                         void* k_cache, void* v_cache, const pkv_cache_desc* cache, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num_pairs < 0 || block_bytes(cache) >= pkv::kMoveMaxBlockBytes) return PKV_ERR_SHAPE;
  if (num_pairs == 0) return PKV_OK;
  if (!src_ids || !dst_ids || !k_cache || !v_cache) return PKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_SHAPE;
  hipError_t e = pkv::launch_move_blocks(k_cache, v_cache, src_ids, k_cache, v_cache, dst_ids, num_pairs,
                                         block_bytes(cache), cache->num_blocks, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_swap_out(const int32_t* ids, int32_t num, const void* k_cache, const void* v_cache,
                      const pkv_cache_desc* cache, void* k_buf, void* v_buf, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num < 0 || block_bytes(cache) >= pkv::kMoveMaxBlockBytes) return PKV_ERR_SHAPE;
  if (num == 0) return PKV_OK;
  if (!ids || !k_cache || !v_cache || !k_buf || !v_buf) return PKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_buf) || !aligned16(v_buf))
    return PKV_ERR_SHAPE;
  void *kd, *vd;
  if (device_view(k_buf, &kd) || device_view(v_buf, &vd)) return PKV_ERR_SHAPE;
  hipError_t e = pkv::launch_move_blocks(k_cache, v_cache, ids, kd, vd, nullptr, num,
                                         block_bytes(cache), cache->num_blocks, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_swap_in(const int32_t* ids, int32_t num, const void* k_buf, const void* v_buf,
                     void* k_cache, void* v_cache, const pkv_cache_desc* cache, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num < 0 || block_bytes(cache) >= pkv::kMoveMaxBlockBytes) return PKV_ERR_SHAPE;
  if (num == 0) return PKV_OK;
  if (!ids || !k_cache || !v_cache || !k_buf || !v_buf) return PKV_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_buf) || !aligned16(v_buf))
    return PKV_ERR_SHAPE;
  void *kd, *vd;
  if (device_view(const_cast<void*>(k_buf), &kd) || device_view(const_cast<void*>(v_buf), &vd))
    return PKV_ERR_SHAPE;
  hipError_t e = pkv::launch_move_blocks(kd, vd, nullptr, k_cache, v_cache, ids, num,
                                         block_bytes(cache), cache->num_blocks, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// ---- input checks ------------------------------------------------------------------
// The result must be device memory the kernels can update with device-scope atomics: a
// NULL or misaligned pointer, or one the runtime does not know as device memory, is
// refused before anything is launched.
static int check_result_ptr(pkv_check_result* result) {
  if (!result) return PKV_ERR_NULL;
  if ((uintptr_t)result & 7u) return PKV_ERR_SHAPE;
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, result) != hipSuccess) {
    (void)hipGetLastError();
    return PKV_ERR_SHAPE;
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Host-side checks shared by the attention checks: the sizes a call of that kind refuses.
static int check_attention_sizes(int32_t num_seqs, const pkv_cache_desc* cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len) {
  int st = check_cache(cache);
  if (st) return st;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size < max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_NULL;
  return PKV_OK;
}

static pkv::SeqCheckArgs seq_check_args(int32_t num_seqs, const pkv_cache_desc* cache, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* context_lens,
                                        int32_t max_context_len) {
  pkv::SeqCheckArgs a = {};
  a.num_seqs = num_seqs;
  a.num_blocks = cache->num_blocks;
  a.block_size = cache->block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  return a;
}

int paged_kv_check_slots(const int64_t* slot_mapping, int32_t num_tokens, const pkv_cache_desc* cache,
                         pkv_check_result* result, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num_tokens < 0) return PKV_ERR_SHAPE;
  if (num_tokens > 0 && !slot_mapping) return PKV_ERR_NULL;
  if ((st = check_result_ptr(result))) return st;
  pkv::DupCheckArgs a = {};
  a.n = num_tokens;
  a.rows = cache->num_blocks * cache->block_size;
  a.slots = slot_mapping;
  hipError_t e = pkv::launch_check_dups(pkv::kDupSlots, a, result, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_check_positions(const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                             int32_t num_seqs, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const pkv_cache_desc* cache, pkv_check_result* result, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if (num_tokens > 0 && (!seq_ids || !positions || (num_seqs > 0 && !block_tables))) return PKV_ERR_NULL;
  if ((st = check_result_ptr(result))) return st;
  pkv::DupCheckArgs a = {};
  a.n = num_tokens;
  a.rows = cache->num_blocks * cache->block_size;
  a.seq_ids = seq_ids;
  a.positions = positions;
  a.num_seqs = num_seqs;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.block_size = cache->block_size;
  hipError_t e = pkv::launch_check_dups(pkv::kDupPositions, a, result, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_attention_check_decode(int32_t num_seqs, const pkv_cache_desc* cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int32_t window, int32_t sinks,
                                 pkv_check_result* result, hipStream_t stream) {
  int st = check_attention_sizes(num_seqs, cache, block_tables, max_blocks_per_seq, context_lens, max_context_len);
  if (st) return st;
  if (window < 0 || sinks < 0) return PKV_ERR_SHAPE;
  if ((st = check_result_ptr(result))) return st;
  pkv::SeqCheckArgs a = seq_check_args(num_seqs, cache, block_tables, max_blocks_per_seq, context_lens,
                                       max_context_len);
  a.window = window;
  a.sinks = sinks;
  hipError_t e = pkv::launch_check_seqs(a, nullptr, result, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_attention_check_shared_prefix(int32_t num_seqs, const pkv_cache_desc* cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        const int32_t* group_starts, int32_t num_groups,
                                        int32_t max_group_size, const int32_t* prefix_lens,
                                        int32_t max_prefix_len, pkv_check_result* result,
                                        hipStream_t stream) {
  int st = check_attention_sizes(num_seqs, cache, block_tables, max_blocks_per_seq, context_lens, max_context_len);
  if (st) return st;
  if (num_seqs > 0) {
    if (num_groups < 1 || num_groups > num_seqs || max_group_size < 1 || max_prefix_len < 0) return PKV_ERR_SHAPE;
    if (max_prefix_len % cache->block_size != 0 || max_prefix_len > max_context_len) return PKV_ERR_SHAPE;
    if (!group_starts || !prefix_lens) return PKV_ERR_NULL;
  }
  if ((st = check_result_ptr(result))) return st;
  pkv::SeqCheckArgs a = seq_check_args(num_seqs, cache, block_tables, max_blocks_per_seq, context_lens,
                                       max_context_len);
  pkv::GroupCheckArgs g = {};
  g.num_seqs = num_seqs;
  g.num_groups = num_groups;
  g.max_group_size = max_group_size;
  g.max_prefix_len = max_prefix_len;
  g.block_size = cache->block_size;
  g.max_blocks_per_seq = max_blocks_per_seq;
  g.group_starts = group_starts;
  g.prefix_lens = prefix_lens;
  g.context_lens = context_lens;
  g.block_tables = block_tables;
  hipError_t e = pkv::launch_check_seqs(a, &g, result, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_attention_check_prefill(int32_t num_seqs, const int32_t* cu_q, int32_t max_q_len,
                                  const pkv_cache_desc* cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, pkv_check_result* result, hipStream_t stream) {
  int st = check_attention_sizes(num_seqs, cache, block_tables, max_blocks_per_seq, context_lens, max_context_len);
  if (st) return st;
  if (max_q_len < 0 || max_q_len > max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs > 0 && !cu_q) return PKV_ERR_NULL;
  if ((st = check_result_ptr(result))) return st;
  pkv::SeqCheckArgs a = seq_check_args(num_seqs, cache, block_tables, max_blocks_per_seq, context_lens,
                                       max_context_len);
  a.cu_q = cu_q;
  a.max_q_len = max_q_len;
  hipError_t e = pkv::launch_check_seqs(a, nullptr, result, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_kv_check_block_ids(const int32_t* src_ids, const int32_t* dst_ids, int32_t num,
                             const pkv_cache_desc* cache, pkv_check_result* result, hipStream_t stream) {
  int st = check_cache(cache);
  if (st) return st;
  if (num < 0) return PKV_ERR_SHAPE;
  if (num > 0 && !dst_ids) return PKV_ERR_NULL;
  if ((st = check_result_ptr(result))) return st;
  pkv::DupCheckArgs a = {};
  a.n = num;
  a.rows = cache->num_blocks;
  a.src_ids = src_ids;
  a.dst_ids = dst_ids;
  hipError_t e = pkv::launch_check_dups(pkv::kDupBlocks, a, result, stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t paged_attention_schedule(const pkv_cache_desc* cache, pkv_dtype q_dtype,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_size, int32_t* partition_out,
                                 int32_t* workers_out) {
  int st = check_decode_shape(cache, q_dtype, q_dtype, num_seqs, num_q_heads, max_context_len);
  if (st) return st;
  Plan plan;
  st = plan_decode(cache, q_dtype, num_seqs, num_q_heads, max_context_len, partition_size, &plan);
  if (st) return st;
  if (partition_out) *partition_out = plan.partition;
  if (workers_out) *workers_out = plan.workers;
  return plan.mode;
}

size_t paged_attention_workspace_size(const pkv_cache_desc* cache, pkv_dtype q_dtype,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_context_len, int32_t partition_size) {
  if (check_decode_shape(cache, q_dtype, q_dtype, num_seqs, num_q_heads, max_context_len)) return 0;
  if (num_seqs == 0) return 0;
  Plan plan;
  if (plan_decode(cache, q_dtype, num_seqs, num_q_heads, max_context_len, partition_size, &plan))
    return 0;
  return plan.ws_bytes;
}

int paged_attention_decode(const void* q, pkv_dtype q_dtype, int32_t num_seqs,
                           int32_t num_q_heads, const void* k_cache, const void* v_cache,
                           const pkv_cache_desc* cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, float scale, void* out,
                           pkv_dtype out_dtype, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return paged_attention_decode_window(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache,
                                       block_tables, max_blocks_per_seq, context_lens, max_context_len,
                                       0, 0, scale, out, out_dtype, partition_size, workspace,
                                       workspace_bytes, stream);
}

int paged_attention_decode_window(const void* q, pkv_dtype q_dtype, int32_t num_seqs,
                                  int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                  const pkv_cache_desc* cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t window, int32_t sinks, float scale,
                                  void* out, pkv_dtype out_dtype, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_decode_call(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                             max_blocks_per_seq, context_lens, max_context_len, window, sinks, out,
                             out_dtype);
  if (st || num_seqs == 0) return st;
  Plan plan;
  st = plan_decode(cache, q_dtype, num_seqs, num_q_heads, max_context_len, partition_size, &plan);
  if (st) return st;
  if (plan.ws_bytes) {
    if (!workspace) return PKV_ERR_NULL;
    if (workspace_bytes < plan.ws_bytes || ((uintptr_t)workspace & 255u)) return PKV_ERR_WORKSPACE;
  }
  return run_decode(plan, q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                    max_blocks_per_seq, context_lens, max_context_len, window, sinks, scale, out, out_dtype,
                    workspace, stream);
}

int paged_attention_decode_noalloc(const void* q, pkv_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                                   const void* k_cache, const void* v_cache, const pkv_cache_desc* cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t max_context_len, float scale,
                                   void* out, pkv_dtype out_dtype, int32_t partition_size, hipStream_t stream) {
  int st = check_decode_call(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                             max_blocks_per_seq, context_lens, max_context_len, 0, 0, out, out_dtype);
  if (st || num_seqs == 0) return st;
  Plan plan;
  st = plan_decode(cache, q_dtype, num_seqs, num_q_heads, max_context_len, partition_size, &plan);
  if (st) return st;
  if (plan.ws_bytes > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
  void* ws = nullptr;
  if (plan.ws_bytes) {
    st = scratch_for_current_device(stream, &ws);
    if (st) return st;
  }
  return run_decode(plan, q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                    max_blocks_per_seq, context_lens, max_context_len, 0, 0, scale, out, out_dtype, ws, stream);
}


size_t paged_attention_shared_prefix_workspace_size(const pkv_cache_desc* cache, pkv_dtype q_dtype,
                                                    int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t max_context_len, int32_t num_groups,
                                                    int32_t max_group_size, int32_t max_prefix_len) {
  if (check_decode_shape(cache, q_dtype, q_dtype, num_seqs, num_q_heads, max_context_len)) return 0;
  if (num_seqs == 0) return 0;
  PrefixPlan plan;
  if (plan_prefix(cache, q_dtype, num_seqs, num_q_heads, max_context_len, num_groups, max_group_size,
                  max_prefix_len, &plan))
    return 0;
  return plan.ws_bytes;
}

int paged_attention_decode_shared_prefix(
    const void* q, pkv_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
    const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
    const int32_t* group_starts, int32_t num_groups, int32_t max_group_size, const int32_t* prefix_lens,
    int32_t max_prefix_len, float scale, void* out, pkv_dtype out_dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  int st = check_decode_shape(cache, q_dtype, out_dtype, num_seqs, num_q_heads, max_context_len);
  if (st) return st;
  if (max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size < max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  PrefixPlan plan;
  st = plan_prefix(cache, q_dtype, num_seqs, num_q_heads, max_context_len, num_groups, max_group_size,
                   max_prefix_len, &plan);
  if (st) return st;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !group_starts ||
      !prefix_lens || !workspace)
    return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_SHAPE;
  if (workspace_bytes < plan.ws_bytes || ((uintptr_t)workspace & 255u)) return PKV_ERR_WORKSPACE;

  float* pre_part = (float*)((char*)workspace + plan.sk.ws_bytes);
  if (max_prefix_len > 0) {
    pkv::RowsArgs p = rows_args(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                                max_blocks_per_seq, scale, plan.tiles, stream);
    p.group_starts = group_starts;
    p.prefix_lens = prefix_lens;
    p.pre_part = pre_part;
    p.splits = plan.splits;
    hipError_t e = pkv::launch_prefix(p, num_groups);
    if (e == hipErrorInvalidValue) return PKV_ERR_SHAPE;
    if (e != hipSuccess) return PKV_ERR_LAUNCH;
  }

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
  a.kv_stream = 1;  // the suffixes are each sequence's own blocks
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.scale = scale;
  a.window = 0;
  a.sinks = 0;
  a.out = out;
  a.out_dtype = out_dtype;
  a.partition = 0;
  a.num_partitions = 0;
  a.ws_m = a.ws_l = a.ws_acc = nullptr;
  a.sk_workers = plan.sk.waves;
  a.sk_count = (int32_t*)workspace;
  a.sk_part = (float*)((char*)workspace + pkv::kWsHeaderBytes);
  a.seq_begin = prefix_lens;
  a.pre_part = pre_part;
  a.pre_splits = plan.splits;
  hipError_t e = pkv::launch_decode_streamk(a, stream);
  if (e == hipErrorInvalidValue) return PKV_ERR_SHAPE;
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int paged_attention_prefill(const void* q, pkv_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                            const int32_t* cu_q, int32_t max_q_len, const void* k_cache, const void* v_cache,
                            const pkv_cache_desc* cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                            float scale, void* out, pkv_dtype out_dtype, hipStream_t stream) {
  int st = check_decode_shape(cache, q_dtype, out_dtype, num_seqs, num_q_heads, max_context_len);
  if (st) return st;
  if (cache->dtype == PKV_F32) return PKV_ERR_DTYPE;  // 16-bit and fp8 caches (queries checked as decode)
  if (max_q_len < 0 || max_q_len > max_context_len || max_blocks_per_seq <= 0) return PKV_ERR_SHAPE;
  if ((int64_t)max_blocks_per_seq * cache->block_size < max_context_len) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || max_q_len == 0) return PKV_OK;
  if (!q || !cu_q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_ERR_SHAPE;
  const int32_t G = num_q_heads / cache->num_kv_heads;
  const int64_t tiles = ((int64_t)max_q_len * G + pkv::kPrefillRows - 1) / pkv::kPrefillRows;
  if (tiles * num_seqs * cache->num_kv_heads > 0x7fffffff) return PKV_ERR_SHAPE;
  pkv::RowsArgs p = rows_args(q, q_dtype, num_seqs, num_q_heads, k_cache, v_cache, cache, block_tables,
                              max_blocks_per_seq, scale, (int32_t)tiles, stream);
  p.cu_q = cu_q;
  p.context_lens = context_lens;
  p.out = out;
  p.out_dtype = out_dtype;
  hipError_t e = pkv::launch_prefill(p);
  if (e == hipErrorInvalidValue) return PKV_ERR_SHAPE;
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
