// Input checks for gfx950: the preconditions the hot-path calls leave unchecked on the
// device, tested on the caller's index arrays alone (never a cache).  Each check runs in
// order on one stream: a launch that clears the result, the launches that test the entries
// (one, or three for the shared-prefix rules), and one that turns the result's accumulators
// into the reported form.
//
// The rules follow from what the calls do with their indices:
//   * a slot names one cache row, block_tables[s][p / B] * B + p % B ("Optimizacion de
//     Inferencia LLM", section "PagedAttention: Conceptos de SO...", get_physical_block),
//     and two tokens writing one row in one call race;
//   * a decode or prefill reads the physical block of every logical block holding a token
//     it attends to ("PagedAttention por dentro...", sections "La tabla de paginas (block
//     table)", "Sliding window attention" and "StreamingLLM...: los attention sinks"),
//     so those IDs must lie in the pool;
//   * sequences sharing a prefix point their tables at the same blocks ("La despensa por
//     casilleros", section "Prefix caching: compartir casilleros con copy-on-write");
//   * copy-on-write copies into a fresh block ("PagedAttention por dentro...", section
//     "Copy-on-write para sampling paralelo"), and a swapped-in block receives one row
//     (section "Estrategia 2: swap").
//
// Accumulation: the caller's 24-byte result is used as {flag, key, count}.  A violation
// of rule `code` at `index` is the key (code << 56) | index; the smallest key wins (an
// atomic minimum: the lowest code, then its lowest index) and every violation adds one to
// the count.  `flag` marks a broken grouping for the shared-prefix rules that need a
// valid one.  Atomics go through vector memory instructions at device scope; a kernel
// boundary orders the launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_launch.h"

namespace pkv {

namespace {

struct CheckState {
  int32_t code;   // reported code (written at the end)
  int32_t flag;   // 1: group_starts broke a rule
  uint64_t key;   // smallest (code << 56) | index, or kNoKey
  uint64_t count; // violations
};
static_assert(sizeof(CheckState) == 24, "layout of pkv_check_result");

constexpr uint64_t kNoKey = ~0ull;
constexpr uint64_t kIndexMask = (1ull << 56) - 1;
constexpr int kCheckThreads = 256;

enum : int {
  kDuplicateSlot = 1,
  kSeqId = 2,
  kContextLen = 3,
  kBlockId = 4,
  kGroupStarts = 5,
  kPrefixLen = 6,
  kPrefixBlocks = 7,
  kQueryRows = 8,
  kBlockPair = 9
};

__device__ __forceinline__ void report(CheckState* r, int code, uint64_t index) {
  __hip_atomic_fetch_add(&r->count, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_fetch_min(&r->key, ((uint64_t)code << 56) | (index & kIndexMask), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void check_init_kernel(CheckState* r) {
  if (threadIdx.x != 0) return;
  r->code = 0;
  r->flag = 0;
  r->key = kNoKey;
  r->count = 0;
}

// key -> (code, index); index -1 and code 0 when nothing was reported.
__global__ void check_finish_kernel(CheckState* r) {
  if (threadIdx.x != 0) return;
  const uint64_t key = __hip_atomic_load(&r->key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r->code = key == kNoKey ? 0 : (int32_t)(key >> 56);
  r->flag = 0;
  r->key = key == kNoKey ? ~0ull : (key & kIndexMask);  // ~0 reads as index -1
}

// ---- per-sequence rules: CONTEXT_LEN, QUERY_ROWS, BLOCK_ID ---------------------------
// One wave per sequence (four per workgroup).  The table entries a sequence reads are
// those of blocks holding an attended token; context_lens[s] <= max_context_len <=
// max_blocks * B (the latter checked on the host) keeps them inside its row.
__global__ void __launch_bounds__(kCheckThreads) check_seqs_kernel(SeqCheckArgs a, CheckState* r) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * (kCheckThreads / 64) + (threadIdx.x >> 6);
  if (s >= a.num_seqs) return;
  const int32_t ctx = a.context_lens[s];
  bool reads = true;
  if (ctx < 0 || ctx > a.max_context_len) {
    if (lane == 0) report(r, kContextLen, (uint64_t)s);
    reads = false;
  }
  if (a.cu_q) {
    const int64_t n = (int64_t)a.cu_q[s + 1] - a.cu_q[s];
    const bool bad = (s == 0 && a.cu_q[0] != 0) || n < 0 || n > a.max_q_len || n > ctx;
    if (bad && lane == 0) report(r, kQueryRows, (uint64_t)s);
    if (bad || n < 1) reads = false;
  }
  if (!reads) return;
  const int B = a.block_size;
  const int nb = (ctx + B - 1) / B;
  const int32_t* row = a.block_tables + s * a.max_blocks_per_seq;
  for (int j = lane; j < nb; j += 64) {
    if (a.window > 0) {
      // block j holds positions [jB, min((j+1)B, ctx)); attended: >= ctx - window or < sinks
      const int64_t lo = (int64_t)j * B;
      const int64_t last = ((int64_t)(j + 1) * B < ctx ? (int64_t)(j + 1) * B : (int64_t)ctx) - 1;
      if (!(last >= (int64_t)ctx - a.window || lo < a.sinks)) continue;
    }
    const int32_t id = row[j];
    if (id < 0 || id >= a.num_blocks) report(r, kBlockId, (uint64_t)s * a.max_blocks_per_seq + j);
  }
}

// ---- shared-prefix grouping: GROUP_STARTS (one thread per entry) ---------------------
__global__ void __launch_bounds__(kCheckThreads) check_group_starts_kernel(GroupCheckArgs a, CheckState* r) {
  const int64_t j = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  if (j > a.num_groups) return;
  const int64_t v = a.group_starts[j];
  bool bad = v < 0 || v > a.num_seqs || (j == 0 && v != 0) || (j == a.num_groups && v != a.num_seqs);
  if (j < a.num_groups) {
    const int64_t size = (int64_t)a.group_starts[j + 1] - v;
    bad = bad || size < 0 || size > a.max_group_size;
  }
  if (bad) {
    report(r, kGroupStarts, (uint64_t)j);
    __hip_atomic_store(&r->flag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- PREFIX_LEN, PREFIX_BLOCKS: one workgroup per group, after the grouping check ----
// With the grouping valid every start lies in [0, num_seqs] and the groups are in order,
// so the members read are sequences; prefix_lens[f] <= max_prefix_len <= max_context_len
// <= max_blocks * B keeps the compared entries inside the rows.
__global__ void __launch_bounds__(kCheckThreads) check_prefix_kernel(GroupCheckArgs a, CheckState* r) {
  if (__hip_atomic_load(&r->flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return;
  const int32_t f = a.group_starts[blockIdx.x];
  const int32_t e = a.group_starts[blockIdx.x + 1];
  if (e <= f) return;
  const int B = a.block_size;
  const int32_t p0 = a.prefix_lens[f];
  for (int32_t s = f + (int32_t)threadIdx.x; s < e; s += kCheckThreads) {
    const int32_t p = a.prefix_lens[s];
    if (p < 0 || p % B != 0 || p > a.max_prefix_len || p > a.context_lens[s] || p != p0)
      report(r, kPrefixLen, (uint64_t)s);
  }
  if (p0 < 0 || p0 % B != 0 || p0 > a.max_prefix_len) return;
  const int64_t nb0 = p0 / B;
  const int64_t total = (int64_t)(e - f - 1) * nb0;
  const int32_t* first = a.block_tables + (int64_t)f * a.max_blocks_per_seq;
  for (int64_t k = threadIdx.x; k < total; k += kCheckThreads) {
    const int64_t s = f + 1 + k / nb0;
    const int64_t b = k % nb0;
    if (a.block_tables[s * a.max_blocks_per_seq + b] != first[b])
      report(r, kPrefixBlocks, (uint64_t)(s * a.max_blocks_per_seq + b));
  }
}

// ---- duplicate rules: DUPLICATE_SLOT (and SEQ_ID), BLOCK_PAIR --------------------------
// Each entry's key is the cache row (or block) it writes, -1 when it writes nothing.  An
// entry breaks the rule when an earlier entry has its key, or (block pairs with sources)
// when any active pair reads from its destination.  Every workgroup compares its 256
// entries against tiles of 256 staged in LDS: quadratic in the entry count.
template <int MODE>
__device__ __forceinline__ int64_t dup_key(const DupCheckArgs& a, int64_t i, int64_t* src_key) {
  *src_key = -1;
  if (MODE == kDupSlots) {
    const int64_t v = a.slots[i];
    return v >= 0 && v < a.rows ? v : -1;
  } else if (MODE == kDupPositions) {
    const int32_t s = a.seq_ids[i], p = a.positions[i];
    if (s < 0 || p < 0 || s >= a.num_seqs) return -1;
    const int32_t j = p / a.block_size;
    if (j >= a.max_blocks_per_seq) return -1;
    const int64_t slot = (int64_t)a.block_tables[(int64_t)s * a.max_blocks_per_seq + j] * a.block_size +
                         p % a.block_size;
    return slot >= 0 && slot < a.rows ? slot : -1;
  } else {
    const int64_t d = a.dst_ids[i];
    const int64_t sv = a.src_ids ? (int64_t)a.src_ids[i] : 0;
    const bool active = d >= 0 && d < a.rows && sv >= 0 && sv < a.rows;
    if (!active) return -1;
    if (a.src_ids) *src_key = sv;
    return d;
  }
}

template <int MODE>
__global__ void __launch_bounds__(kCheckThreads) check_dups_kernel(DupCheckArgs a, CheckState* r) {
  __shared__ int64_t keys[kCheckThreads];
  __shared__ int64_t srcs[kCheckThreads];
  const int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x;
  int64_t mine = -1, unused;
  if (i < a.n) {
    mine = dup_key<MODE>(a, i, &unused);
    if (MODE == kDupPositions && a.seq_ids[i] >= a.num_seqs) report(r, kSeqId, (uint64_t)i);
  }
  const bool sources = MODE == kDupBlocks && a.src_ids;
  // earlier entries only, unless sources are compared too (then every tile)
  const int64_t end = sources ? a.n : ((int64_t)(blockIdx.x + 1) * kCheckThreads < a.n
                                            ? (int64_t)(blockIdx.x + 1) * kCheckThreads : a.n);
  bool bad = false;
  for (int64_t t0 = 0; t0 < end; t0 += kCheckThreads) {
    const int64_t t = t0 + threadIdx.x;
    int64_t sk = -1;
    keys[threadIdx.x] = t < a.n ? dup_key<MODE>(a, t, &sk) : -1;
    srcs[threadIdx.x] = sk;
    __syncthreads();
    if (mine >= 0) {
      const int m = (int)(a.n - t0 < kCheckThreads ? a.n - t0 : kCheckThreads);
      for (int u = 0; u < m; ++u) {
        bad = bad || (t0 + u < i && keys[u] == mine) || (sources && srcs[u] == mine);
      }
    }
    __syncthreads();
  }
  if (bad) report(r, MODE == kDupBlocks ? kBlockPair : kDuplicateSlot, (uint64_t)i);
}

unsigned blocks_for(int64_t n, int64_t per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_check_seqs(const SeqCheckArgs& a, const GroupCheckArgs* groups, void* result,
                             hipStream_t stream) {
  CheckState* r = (CheckState*)result;
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, r);
  if (a.num_seqs > 0)
    hipLaunchKernelGGL(check_seqs_kernel, dim3(blocks_for(a.num_seqs, kCheckThreads / 64)), dim3(kCheckThreads),
                       0, stream, a, r);
  if (groups && a.num_seqs > 0) {
    hipLaunchKernelGGL(check_group_starts_kernel, dim3(blocks_for((int64_t)groups->num_groups + 1, kCheckThreads)),
                       dim3(kCheckThreads), 0, stream, *groups, r);
    hipLaunchKernelGGL(check_prefix_kernel, dim3((unsigned)groups->num_groups), dim3(kCheckThreads), 0, stream,
                       *groups, r);
  }
  hipLaunchKernelGGL(check_finish_kernel, dim3(1), dim3(64), 0, stream, r);
  return hipGetLastError();
}

hipError_t launch_check_dups(int mode, const DupCheckArgs& a, void* result, hipStream_t stream) {
  CheckState* r = (CheckState*)result;
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, r);
  if (a.n > 0) {
    const dim3 grid(blocks_for(a.n, kCheckThreads)), block(kCheckThreads);
    if (mode == kDupSlots)
      hipLaunchKernelGGL(check_dups_kernel<kDupSlots>, grid, block, 0, stream, a, r);
    else if (mode == kDupPositions)
      hipLaunchKernelGGL(check_dups_kernel<kDupPositions>, grid, block, 0, stream, a, r);
    else
      hipLaunchKernelGGL(check_dups_kernel<kDupBlocks>, grid, block, 0, stream, a, r);
  }
  hipLaunchKernelGGL(check_finish_kernel, dim3(1), dim3(64), 0, stream, r);
  return hipGetLastError();
}

}  // namespace pkv
