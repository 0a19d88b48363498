// Internal launcher interface between the C ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

struct WriteArgs {
  const int64_t* slot_mapping;  // given slots; or, when seq_ids is set, slots resolved in the
  const int32_t* seq_ids;       // write kernel from seq_ids / positions / block_tables (and
  const int32_t* positions;     // stored to slot_out unless it is null)
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  int64_t* slot_out;
  int32_t num_tokens;
  const void* k;
  const void* v;
  int src_dtype;
  void* k_cache;
  void* v_cache;
  int cache_dtype;
  int32_t num_kv_heads, head_dim, block_size;
  int64_t num_blocks;
  float k_scale, v_scale;
};

struct DecodeArgs {
  const void* q;
  int q_dtype;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int cache_dtype;
  const void* k_cache;
  const void* v_cache;
  float k_scale, v_scale;
  int32_t kv_stream;       // 1: K/V read with the streaming (nontemporal) policy
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t max_context_len;
  float scale;
  // sliding window with attention sinks: window > 0 attends to the last `window`
  // tokens of each context and its first `sinks`; window == 0 to every token
  int32_t window, sinks;
  void* out;
  int out_dtype;
  int32_t partition;       // tokens per partition (> 0)
  int32_t num_partitions;  // grid extent; 1 = single pass (no workspace)
  float* ws_m;             // [N][H_q][P] running max (log2 domain), split mode only
  float* ws_l;             // [N][H_q][P] softmax denominators
  float* ws_acc;           // [N][H_q][P][D] unnormalised outputs
  // balanced schedule
  int32_t sk_workers;      // waves in the launch
  int32_t* sk_count;       // [workgroups] arrival counters: zero on entry, zero on exit
  float* sk_part;          // [2 * workgroups] partials: m[GP], l[GP], (16-byte aligned) acc[GP][D]
  // suffix pass of the shared-prefix decode (balanced schedule only; null otherwise)
  const int32_t* seq_begin;  // [N] tokens of each context already attended (a multiple of 16)
  const float* pre_part;     // [N][H_q][pre_splits][4 + D]: m, l, pad, pad, acc
  int32_t pre_splits;
};

// Many query rows against one paged token range on the matrix cores (mfma_rows.hip):
// the shared-prefix pass (partials of every group's shared prefix) and chunked prefill.
struct RowsArgs {
  const void* q;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim, block_size;
  int cache_dtype, q_dtype;
  float k_scale, v_scale;  // fp8 caches: value = code * scale (1 otherwise)
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  float scale;
  int32_t tiles;                // kPrefixRows-row tiles per group / kPrefillRows-row tiles per sequence
  hipStream_t stream;
  // shared prefix
  const int32_t* group_starts;  // [groups + 1]
  const int32_t* prefix_lens;   // [N]
  float* pre_part;              // [N][H_q][splits][4 + D]: m, l, pad, pad, acc
  int32_t splits;               // slices of each prefix's chunks
  // chunked prefill
  const int32_t* cu_q;          // [N + 1]: query rows of sequence s are cu_q[s] .. cu_q[s+1]-1
  const int32_t* context_lens;  // [N], counting the chunk
  void* out;                    // [rows][H_q][D]
  int out_dtype;
};
constexpr int kPrefixRows = 64;    // query rows per workgroup of the rows kernel: shared-prefix pass
constexpr int kPrefillRows = 128;  // the same for chunked prefill
hipError_t launch_prefix(const RowsArgs& a, int num_groups);
hipError_t launch_prefill(const RowsArgs& a);

// Whole-block moves (copy-on-write, swap): pair i moves block src_ids[i] (row i when
// src_ids is null) of each of the K and V sources to block dst_ids[i] (row i when
// dst_ids is null) of the destinations; a negative ID skips the pair.
// An ID array's entries address blocks [0, num_blocks) of that side's cache; the others
// are skipped.  A null ID array means row i of a contiguous buffer.
constexpr int64_t kMoveMaxBlockBytes = ((int64_t)1 << 31) - 32768;  // 32-bit offsets with a round's headroom
hipError_t launch_move_blocks(const void* k_src, const void* v_src, const int32_t* src_ids, void* k_dst,
                              void* v_dst, const int32_t* dst_ids, int32_t num, int64_t block_bytes,
                              int64_t num_blocks, hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* seq_ids, const int32_t* positions, int32_t n,
                               const int32_t* block_tables, int32_t max_blocks,
                               int32_t block_size, int64_t* slots, hipStream_t stream);
hipError_t launch_kv_write(const WriteArgs& a, hipStream_t stream);
// Return hipErrorInvalidValue for an unsupported combination (checked earlier by the ABI).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);          // fixed partitions
hipError_t launch_decode_streamk(const DecodeArgs& a, hipStream_t stream);  // balanced

// Balanced schedule: one workgroup per resident slot of the chosen kernel on the
// current device (a full MI355X if no device is visible).  streamk_plan fills the
// waves of the launch and the workspace it needs; it returns 0, or -1 for an
// unsupported combination or a kernel that does not fit a CU (e.g. too many sequences
// for its LDS prefix array).
constexpr int kStreamKMaxSeqs = 8191;
constexpr int kStreamKMaxGroups = 8192;
struct SkPlan {
  int waves;
  size_t ws_bytes;
};
int pad_group(int G);
int streamk_plan(int cache_dtype, int q_dtype, int head_dim, int group, int num_seqs, bool kv_stream,
                 bool pre, SkPlan* out);

// Every workspace starts with a header of arrival counters (one int per workgroup of
// a balanced launch) that is zero before the first call and that every call leaves
// zero; no schedule stores anything else there.  Arrays after it are 256-byte aligned.
constexpr size_t kWsHeaderBytes = (size_t)kStreamKMaxGroups * sizeof(int32_t);
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t ws_ml_bytes(int64_t n, int64_t hq, int64_t parts) {
  return align256((size_t)(n * hq * parts) * sizeof(float));
}
inline size_t ws_total_bytes(int64_t n, int64_t hq, int64_t d, int64_t parts) {
  return kWsHeaderBytes + 2 * ws_ml_bytes(n, hq, parts) +
         align256((size_t)(n * hq * parts * d) * sizeof(float));
}

// ---- input checks (check.hip); `result` is the caller's pkv_check_result ----
struct SeqCheckArgs {
  int64_t num_seqs;
  int64_t num_blocks;
  int32_t block_size, max_blocks_per_seq, max_context_len;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t window, sinks;  // decode over a window (window 0: every token)
  const int32_t* cu_q;    // prefill: query rows [num_seqs + 1]; null otherwise
  int32_t max_q_len;
};
struct GroupCheckArgs {  // shared-prefix grouping
  int32_t num_seqs, num_groups, max_group_size, max_prefix_len, block_size, max_blocks_per_seq;
  const int32_t* group_starts;
  const int32_t* prefix_lens;
  const int32_t* context_lens;
  const int32_t* block_tables;
};
enum DupMode { kDupSlots = 0, kDupPositions = 1, kDupBlocks = 2 };
struct DupCheckArgs {
  int64_t n;     // entries
  int64_t rows;  // slots: num_blocks * block_size; block pairs: num_blocks
  const int64_t* slots;
  const int32_t* seq_ids;
  const int32_t* positions;
  int32_t num_seqs, max_blocks_per_seq, block_size;
  const int32_t* block_tables;
  const int32_t* src_ids;  // block pairs: null for swap in
  const int32_t* dst_ids;
};
// CONTEXT_LEN / QUERY_ROWS / BLOCK_ID per sequence, and with `groups` the shared-prefix
// rules; a clear, the checks and the final write of `result`, in order on `stream`.
hipError_t launch_check_seqs(const SeqCheckArgs& a, const GroupCheckArgs* groups, void* result,
                             hipStream_t stream);
hipError_t launch_check_dups(int mode, const DupCheckArgs& a, void* result, hipStream_t stream);

}  // namespace pkv
