/*
 * pagedkv.h -- C ABI of the paged KV cache decode path for AMD MI355X (gfx950).
 *
 * One decode step of one attention layer:
 *   1. paged_kv_slot_mapping  -- resolve (sequence, position) to a cache slot
 *                                through the block table;
 *   2. paged_kv_write         -- store each new token's K and V in its slot;
 *   3. paged_attention_decode -- every query head of the new token attends over
 *                                its sequence's whole cached context, new token
 *                                included, reading K/V through the block table.
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer owned by the caller (allocated by
 *     any HIP allocator, e.g. PyTorch).  The library allocates and frees nothing;
 *     its only global state is a per-device cache of kernel-occupancy queries
 *     (filled on first use, safe under concurrent calls) and the scratch array of
 *     paged_attention_decode_noalloc (below).  Concurrent calls on different streams
 *     are safe as long as they do not write the same memory.
 *   - Every call is asynchronous on `stream` (NULL = the null stream).  Buffers
 *     must stay alive until the caller synchronises.  Host-visible argument
 *     errors are returned before anything is launched; no call synchronises
 *     with the device, so errors inside kernels surface at the caller's next sync.
 *   - Return value: PKV_OK (0) or a negative pkv_status.  No exception crosses
 *     the ABI.  pkv_status_string() names each code.
 *
 * Cache layout (both K and V): [num_blocks][num_kv_heads][block_size][head_dim],
 * row-major.  One (block, KV head) tile is block_size * head_dim contiguous
 * elements, so a 16-token bf16 tile of head_dim 128 is 4 KiB read with 16-byte
 * loads per lane.  Token position p of sequence s lives at physical block
 * block_tables[s][p / block_size], offset p % block_size ("PagedAttention por
 * dentro...", section "La tabla de paginas (block table)"; "Optimizacion de
 * Inferencia LLM", section "PagedAttention: Conceptos de SO...", get_physical_block).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3 /* OCP e4m3fn: bias 7, no infinities, S.1111.111 = NaN, max 448 */
} pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_DTYPE = -2,       /* unsupported dtype or dtype combination */
  PKV_ERR_SHAPE = -3,       /* unsupported head_dim / block_size / group size, or bad sizes */
  PKV_ERR_HEADS = -4,       /* num_q_heads is not a multiple of num_kv_heads */
  PKV_ERR_WORKSPACE = -5,   /* workspace too small, or bad partition size */
  PKV_ERR_LAUNCH = -6,      /* the HIP runtime reported an error at launch */
  PKV_ERR_POOL_EXHAUSTED = -7, /* block pool: fewer free blocks than asked for */
  PKV_ERR_BLOCK_STATE = -8, /* block pool: a block ID out of range, or not allocated */
  PKV_ERR_SCRATCH = -9      /* paged_attention_decode_noalloc: the call needs more scratch
                               than PKV_NOALLOC_SCRATCH_BYTES */
} pkv_status;

/* Every non-empty decode workspace starts with this many bytes of arrival counters,
 * which must be zero before the workspace's first use (e.g. hipMemset once after
 * allocation) and which every paged_attention_decode call leaves zero when it
 * completes.  Nothing else is ever stored there; the rest of the workspace may hold
 * anything on entry. */
#define PKV_WORKSPACE_HEADER_BYTES 32768

/* pkv_cache_desc.flags: the block tables of one decode call may map several
 * sequences to the same physical block (prefix caching: "La despensa por
 * casilleros", section "Prefix caching"; "PagedAttention por dentro...", section
 * "Prefix caching cross-session").  The decode then reads K/V with the ordinary cache policy,
 * so a shared block stays in L2 for its other readers.  Without the flag every
 * K/V byte is assumed to be read once per call and is read with the streaming
 * (nontemporal) policy, which is faster for such data.  Either way the results are
 * identical; only speed differs. */
#define PKV_CACHE_SHARED_BLOCKS 1

/* Describes one layer's paged cache (K and V share it). */
typedef struct {
  int64_t num_blocks;   /* physical blocks in the pool */
  int32_t block_size;   /* tokens per block: 16 or 32 */
  int32_t num_kv_heads; /* H_kv */
  int32_t head_dim;     /* d_h: 64 or 128 */
  int32_t dtype;        /* pkv_dtype of the stored elements */
  float k_scale;        /* fp8 only: stored code * k_scale = K value (1.0 otherwise) */
  float v_scale;        /* fp8 only: stored code * v_scale = V value */
  int32_t flags;        /* 0 or PKV_CACHE_SHARED_BLOCKS; other bits: PKV_ERR_SHAPE */
} pkv_cache_desc;

/*
 * slot_mapping[t] = block_tables[seq_ids[t]][positions[t] / B] * B + positions[t] % B
 * for each of num_tokens tokens; a negative position or sequence ID, or a position
 * whose block index is >= max_blocks_per_seq, gives slot -1 ("skip").
 * Source: "Optimizacion de Inferencia LLM", section "PagedAttention: Conceptos de
 * SO...", BlockTable.get_physical_block.
 *   seq_ids, positions : int32 [num_tokens]
 *   block_tables       : int32 [num_seqs][max_blocks_per_seq]
 *   slot_mapping       : int64 [num_tokens] (output)
 * Precondition (not checked on the device): seq_ids[t] < num_seqs.  num_tokens == 0
 * launches nothing.
 */
int paged_kv_slot_mapping(const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t block_size, int64_t* slot_mapping, hipStream_t stream);

/*
 * Store token t's K and V at cache[slot / B][h][slot % B][:] for every KV head h.
 * Source: "PagedAttention por dentro...", section "La tabla de paginas (block
 * table)" (a new token fills the last block's free slot or the first slot of a
 * freshly appended block); "Capitulo 2", section "Que guarda realmente el KV
 * cache" (the new k_t, v_t join the cached state).
 *   slot_mapping : int64 [num_tokens]; a negative slot, or one >= num_blocks * B,
 *                  skips that token
 *   k, v         : [num_tokens][num_kv_heads][head_dim] of src_dtype (f32/f16/bf16)
 *   k_cache, v_cache : the cache described by `cache`
 * Conversion: same dtype -> bit copy; fp8 cache -> e4m3fn of fl32(fl32(x) / scale)
 * rounded to nearest-even, saturated to +-448, NaN kept NaN.
 * Precondition (not checked on the device): slots unique.
 */
int paged_kv_write(const int64_t* slot_mapping, int32_t num_tokens, const void* k,
                   const void* v, pkv_dtype src_dtype, void* k_cache, void* v_cache,
                   const pkv_cache_desc* cache, hipStream_t stream);

/*
 * Slot resolution and the write in one launch: token t's slot is resolved as by
 * paged_kv_slot_mapping (from seq_ids[t], positions[t] and block_tables) inside the
 * write kernel, and its K and V are stored as by paged_kv_write.  Same sources: the
 * block-table lookup of "Optimizacion de Inferencia LLM", section "PagedAttention:
 * Conceptos de SO..." (get_physical_block) and the append of "PagedAttention por
 * dentro...", section "La tabla de paginas (block table)".
 *   seq_ids, positions : int32 [num_tokens]
 *   block_tables       : int32 [num_seqs][max_blocks_per_seq]
 *   k, v, k_cache, v_cache, cache, src_dtype : as for paged_kv_write
 *   slot_mapping       : int64 [num_tokens] output of the resolved slots (-1 where
 *                        none), or NULL when the caller needs no slots
 * A token with a negative position or sequence ID, a position past the table's row,
 * or a slot outside the cache writes nothing.  Errors as paged_kv_write, plus
 * PKV_ERR_SHAPE for max_blocks_per_seq <= 0.  Preconditions (not checked on the
 * device): seq_ids[t] < num_seqs; resolved slots unique.  num_tokens == 0 launches
 * nothing.  Asynchronous on `stream`; no allocation.
 */
int paged_kv_write_positions(const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                             const int32_t* block_tables, int32_t max_blocks_per_seq, const void* k,
                             const void* v, pkv_dtype src_dtype, void* k_cache, void* v_cache,
                             const pkv_cache_desc* cache, int64_t* slot_mapping, hipStream_t stream);

/*
 * How paged_attention_decode schedules a call with these arguments.  Returns the
 * schedule (0 = one pass per (sequence, KV head), 1 = fixed partitions merged by a
 * second log-sum-exp kernel, 2 = balanced: one workgroup per CU, equal shares of
 * 16-token chunks per wave, partial results merged in the same kernel -- through LDS
 * inside a workgroup, by the last workgroup to finish a context shared between
 * workgroups) or a negative pkv_status.
 * *partition_out gets the tokens per partition (0 for the balanced schedule),
 * *workers_out the waves of a balanced launch (0 otherwise); either may be NULL.
 * The balanced schedule sizes itself for the current device (a full MI355X when
 * no device is visible).
 */
int32_t paged_attention_schedule(const pkv_cache_desc* cache, pkv_dtype q_dtype,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_size, int32_t* partition_out,
                                 int32_t* workers_out);

/* Bytes of device workspace paged_attention_decode needs for these arguments (0 for
 * one pass, or when the arguments are invalid).  Arguments as for
 * paged_attention_decode. */
size_t paged_attention_workspace_size(const pkv_cache_desc* cache, pkv_dtype q_dtype,
                                      int32_t num_seqs, int32_t num_q_heads,
                                      int32_t max_context_len, int32_t partition_size);

/*
 * out[s][h][:] = softmax_t(scale * q[s][h] . K_t) V_t over t = 0 .. context_lens[s]-1,
 * K_t, V_t of KV head h / (num_q_heads / num_kv_heads), read through block_tables.
 * Sources: "Capitulo 2", section "Que guarda realmente el KV cache" (Attn(q_t,
 * [K_{1:t-1}, k_t], [V_{1:t-1}, v_t])); "Optimizacion de Inferencia LLM", sections
 * "El Cuello de Botella..." (softmax(q k^T / sqrt(d_head)) v) and "PagedAttention:
 * Conceptos de SO..." (per-block loads with online-softmax accumulation); "La
 * despensa por casilleros", section "El mecanismo" (gather in logical order).
 *   q            : [num_seqs][num_q_heads][head_dim] of q_dtype
 *   block_tables : int32 [num_seqs][max_blocks_per_seq]; entries past
 *                  ceil(context_lens[s] / B) are never read
 *   context_lens : int32 [num_seqs], counting the new token (already written)
 *   max_context_len : host-side upper bound of context_lens (sizes the grid)
 *   out          : [num_seqs][num_q_heads][head_dim] of out_dtype (f32/f16/bf16)
 *   partition_size : 0 = balanced schedule (up to 8191 sequences; fixed 512-token
 *                    partitions beyond); -1 = one pass per (sequence, KV head);
 *                    else tokens per partition, a positive multiple of block_size;
 *                    partial results are merged by a log-sum-exp pass
 *   workspace    : device scratch of >= paged_attention_workspace_size() bytes,
 *                  256-byte aligned (may be NULL when that size is 0), whose first
 *                  PKV_WORKSPACE_HEADER_BYTES are zero (see above); calls sharing one
 *                  workspace must not overlap (same stream, or synchronised)
 * Supported: head_dim 64 or 128; block_size 16 or 32; group size
 * num_q_heads / num_kv_heads in 1..16; (q, cache) dtypes (f32, f32), (f16, f16),
 * (bf16, bf16), (bf16 or f16, fp8).  Accumulation is fp32; the output is rounded
 * to nearest-even.  context_lens[s] == 0 gives zeros.
 * Preconditions (not checked on the device): 0 <= context_lens[s] <=
 * max_context_len; block IDs in [0, num_blocks) for the entries read.
 */
int paged_attention_decode(const void* q, pkv_dtype q_dtype, int32_t num_seqs,
                           int32_t num_q_heads, const void* k_cache, const void* v_cache,
                           const pkv_cache_desc* cache, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t max_context_len, float scale, void* out,
                           pkv_dtype out_dtype, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * paged_attention_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Computes exactly what paged_attention_decode computes with the same
 * arguments (the same schedules and kernels); the scratch those kernels need (arrival
 * counters and partial results) lives in a file-scope device array of
 * PKV_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds from this call's
 * first use on it until the process ends.  The call allocates nothing.
 *   Arguments: as paged_attention_decode, without workspace / workspace_bytes.
 *   Errors: as paged_attention_decode; PKV_ERR_SCRATCH when the schedule needs more
 *   than PKV_NOALLOC_SCRATCH_BYTES (paged_attention_workspace_size() tells how much:
 *   e.g. more sequences or partitions than fit; use paged_attention_decode then).
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 *   different streams without synchronisation, or from several host threads) race and
 *   give undefined results.  Calls in order on one stream are safe: each call leaves
 *   the array's counters zero, and its first use on a GPU clears them on `stream`.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (16u << 20)
int paged_attention_decode_noalloc(const void* q, pkv_dtype q_dtype, int32_t num_seqs,
                                   int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                   const pkv_cache_desc* cache, const int32_t* block_tables,
                                   int32_t max_blocks_per_seq, const int32_t* context_lens,
                                   int32_t max_context_len, float scale, void* out,
                                   pkv_dtype out_dtype, int32_t partition_size, hipStream_t stream);

/*
 * Decode attention over a sliding window with attention sinks: each query head attends
 * to the last `window` tokens of its context (the new token included) and to the first
 * `sinks` tokens ("PagedAttention por dentro...", section "Sliding window attention":
 * such models attend only to the last K tokens and the engine keeps only the blocks of
 * the active window; section "StreamingLLM...: los attention sinks": the first 4
 * tokens plus a window of the last K).  Every other argument, the workspace size and
 * the schedules are those of paged_attention_decode, which is the window == 0 case.
 *   window : >= 0; 0 = no window (every token, sinks ignored)
 *   sinks  : >= 0; with window > 0, tokens 0 .. sinks-1 are attended as well
 * Block-table entries of blocks holding no attended token are never read (they may
 * name freed blocks).  Returns PKV_ERR_SHAPE for a negative window or sink count.
 */
int paged_attention_decode_window(const void* q, pkv_dtype q_dtype, int32_t num_seqs,
                                  int32_t num_q_heads, const void* k_cache, const void* v_cache,
                                  const pkv_cache_desc* cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t window, int32_t sinks, float scale,
                                  void* out, pkv_dtype out_dtype, int32_t partition_size,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode attention for a batch in which groups of sequences share a prefix of physical
 * blocks -- prefix caching: their block tables point at the same refcounted blocks
 * ("La despensa por casilleros", section "Prefix caching: compartir casilleros con
 * copy-on-write"; "PagedAttention por dentro...", section "Prefix caching cross-session").
 * Computes exactly what paged_attention_decode computes (same contract for every
 * argument it shares with it), reading each group's shared prefix once for the whole
 * group instead of once per sequence: the queries of the group's sequences are stacked
 * as the rows of one matrix product over the prefix tokens (on the matrix cores), each
 * sequence's remaining tokens are streamed as by the balanced schedule, and the two
 * partial softmax results are merged with the log-sum-exp algebra ("Optimizacion de
 * Inferencia LLM", section "PagedAttention: Conceptos de SO..."; online softmax).
 *   group_starts   : int32 [num_groups + 1], ascending, group_starts[0] = 0,
 *                    group_starts[num_groups] = num_seqs; group j is sequences
 *                    group_starts[j] .. group_starts[j+1] - 1
 *   num_groups     : >= 1 (<= num_seqs); a sequence that shares nothing may be a
 *                    group of its own with prefix length 0
 *   max_group_size : host-side upper bound of the group sizes (sizes the grid)
 *   prefix_lens    : int32 [num_seqs]; the first prefix_lens[s] tokens of sequence s
 *                    lie in the blocks its group shares: equal for every sequence of a
 *                    group, a multiple of block_size, <= context_lens[s], and
 *                    block_tables[s][0 .. prefix_lens[s] / block_size) identical across
 *                    the group.  0 = nothing shared.
 *   max_prefix_len : host-side upper bound of prefix_lens (a multiple of block_size)
 *   workspace      : >= paged_attention_shared_prefix_workspace_size() bytes, 256-byte
 *                    aligned, first PKV_WORKSPACE_HEADER_BYTES zero (as for
 *                    paged_attention_decode); never NULL
 * Supported (query, cache): (bf16, bf16), (f16, f16), (bf16 or f16, fp8 e4m3fn with the
 * descriptor's k_scale / v_scale); head_dim, block_size and group size as for
 * paged_attention_decode; up to 8191 sequences.  fp32 caches return PKV_ERR_DTYPE.  The grouping only selects the work split: any grouping that
 * meets the preconditions gives the same attention, to within fp32 rounding order.
 * Preconditions beyond those of paged_attention_decode are not checked on the device.
 */
size_t paged_attention_shared_prefix_workspace_size(const pkv_cache_desc* cache, pkv_dtype q_dtype,
                                                    int32_t num_seqs, int32_t num_q_heads,
                                                    int32_t max_context_len, int32_t num_groups,
                                                    int32_t max_group_size, int32_t max_prefix_len);
int paged_attention_decode_shared_prefix(
    const void* q, pkv_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads, const void* k_cache,
    const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
    const int32_t* group_starts, int32_t num_groups, int32_t max_group_size, const int32_t* prefix_lens,
    int32_t max_prefix_len, float scale, void* out, pkv_dtype out_dtype, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked prefill over the paged cache: each sequence brings a chunk of new query tokens,
 * the last n_s of its context (their K/V already written with paged_kv_write), and query i
 * of the chunk, at position context_lens[s] - n_s + i, attends causally to tokens 0 ..
 * that position ("PagedAttention por dentro...", section "Chunked prefill integrado con
 * paged KV": prompts cut into chunks that run in the same step as decodes, over the same
 * paged KV cache; "Componentes Internos de Servicio de vLLM", section "Chunked prefill
 * protege la cola del TTFT": 512-token chunks by default).  A one-token chunk is a decode.
 *   q            : [rows][num_q_heads][head_dim] of q_dtype, rows = cu_q[num_seqs]
 *   cu_q         : int32 [num_seqs + 1] device, ascending from 0: the query rows of
 *                  sequence s are cu_q[s] .. cu_q[s+1]-1 (n_s = cu_q[s+1] - cu_q[s])
 *   max_q_len    : host-side upper bound of n_s (sizes the grid), <= max_context_len
 *   context_lens : int32 [num_seqs], counting the chunk (n_s <= context_lens[s])
 *   out          : [rows][num_q_heads][head_dim] of out_dtype (f32/f16/bf16)
 * Other arguments as paged_attention_decode.  Supported (query, cache): (bf16, bf16),
 * (f16, f16), (bf16 or f16, fp8 e4m3fn with the descriptor's k_scale / v_scale); head_dim
 * 64 or 128; block_size 16 or 32; group size 1..16.  fp32 caches return PKV_ERR_DTYPE.
 * No workspace.  Preconditions (unchecked on the device):
 * n_s <= max_q_len and n_s <= context_lens[s]; block IDs in range for the tokens read.
 */
int paged_attention_prefill(const void* q, pkv_dtype q_dtype, int32_t num_seqs, int32_t num_q_heads,
                            const int32_t* cu_q, int32_t max_q_len, const void* k_cache, const void* v_cache,
                            const pkv_cache_desc* cache, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                            float scale, void* out, pkv_dtype out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------- block moves ---
 * Whole physical blocks of one layer's K and V caches (block_bytes = num_kv_heads *
 * block_size * head_dim * element bytes each).  IDs are int32 device arrays; an ID
 * outside [0, num_blocks) skips its pair or row.  Asynchronous on `stream`; no
 * allocation.  A block of 2^31 - 32768 bytes or more returns PKV_ERR_SHAPE.
 *
 * Copy-on-write: block src_ids[i] -> block dst_ids[i] in both caches, so a sequence
 * about to write into a block it shares gets a private copy first ("PagedAttention por
 * dentro...", section "Copy-on-write para sampling paralelo": only the last affected
 * block is copied; "La despensa por casilleros", section "Prefix caching...": the block
 * manager copies the block for that branch and only then writes).
 * Precondition (unchecked): destination IDs are distinct from each other and from
 * every source ID (as fresh blocks from pkv_pool_cow are).
 */
int paged_kv_copy_blocks(const int32_t* src_ids, const int32_t* dst_ids, int32_t num_pairs,
                         void* k_cache, void* v_cache, const pkv_cache_desc* cache, hipStream_t stream);

/*
 * Swap out: block ids[i] of each cache -> row i of k_buf / v_buf ([num][block_bytes]);
 * swap in: row i -> block ids[i].  ("PagedAttention por dentro...", section
 * "Estrategia 2: swap": an evicted session's blocks move to CPU RAM and back to VRAM
 * when it resumes.)  The buffers may be device memory or pinned host memory
 * (hipHostMalloc, e.g. torch's pin_memory), in which case the kernel moves the blocks
 * across the host link itself; 16-byte aligned.  A buffer the HIP runtime does not know
 * as device or pinned memory (pageable host memory) returns PKV_ERR_SHAPE before any
 * launch.  Release the swapped-out blocks to the pool only
 * after the stream has finished the swap out, and decode from swapped-in blocks only
 * on the same stream after the swap in (or after synchronising with it).
 * Precondition of swap in (unchecked): its IDs distinct.
 */
int paged_kv_swap_out(const int32_t* ids, int32_t num, const void* k_cache, const void* v_cache,
                      const pkv_cache_desc* cache, void* k_buf, void* v_buf, hipStream_t stream);
int paged_kv_swap_in(const int32_t* ids, int32_t num, const void* k_buf, const void* v_buf,
                     void* k_cache, void* v_cache, const pkv_cache_desc* cache, hipStream_t stream);

/* --------------------------------------------------------------- input checks ---
 * Debugging aids for the preconditions that the calls above leave unchecked on the
 * device (a call that breaks one reads or writes memory the caller did not mean, or
 * races).  Each check reads only the index arrays it is given -- never a cache -- within
 * the bounds its size arguments give, and reports into `result`, a pkv_check_result in
 * device memory (8-byte aligned) that the check initialises itself: a clearing kernel,
 * the check's kernels and a final kernel, in order on `stream`, with no memset, no
 * allocation and no synchronisation, so `result` is valid once the stream has passed the
 * call.  Host-visible argument errors return before
 * anything is launched: PKV_ERR_NULL for a NULL result or a NULL array the check reads,
 * PKV_ERR_SHAPE for negative sizes, the bounds the checked call refuses (a table row
 * shorter than max_context_len, max_q_len above it, the shared-prefix bounds), or a
 * result that is misaligned or not device memory.  Cost: linear in the entries checked, except the
 * duplicate rules, which compare every pair of entries (quadratic in num_tokens or num
 * pairs: a debugging aid, not for the hot path).
 *
 * A violation is one (entry, rule) pair.  `violations` counts them; `code` is the lowest
 * code violated and `index` the lowest index violating it (what an index counts is
 * given per code).  With no violation, code is PKV_CHECK_OK and index -1.
 */
typedef enum {
  PKV_CHECK_OK = 0,
  PKV_CHECK_DUPLICATE_SLOT = 1, /* token t: writes a cache slot an earlier token writes */
  PKV_CHECK_SEQ_ID = 2,         /* token t: seq_ids[t] >= num_seqs */
  PKV_CHECK_CONTEXT_LEN = 3,    /* sequence s: context_lens[s] < 0 or > max_context_len */
  PKV_CHECK_BLOCK_ID = 4,       /* table entry s * max_blocks_per_seq + j read by the call: ID
                                   outside [0, num_blocks) */
  PKV_CHECK_GROUP_STARTS = 5,   /* entry j of group_starts, 0 <= j <= num_groups */
  PKV_CHECK_PREFIX_LEN = 6,     /* sequence s: prefix_lens[s] */
  PKV_CHECK_PREFIX_BLOCKS = 7,  /* table entry s * max_blocks_per_seq + j: a prefix block that
                                   differs from the group's first sequence's */
  PKV_CHECK_QUERY_ROWS = 8,     /* sequence s: its query rows in cu_q */
  PKV_CHECK_BLOCK_PAIR = 9      /* pair or row i: destination repeated, or equal to a source */
} pkv_check_code;

typedef struct {
  int32_t code;       /* pkv_check_code */
  int32_t reserved;   /* 0 after the check */
  int64_t index;      /* -1 when code is PKV_CHECK_OK */
  int64_t violations;
} pkv_check_result;

/* paged_kv_write: token t is *active* when 0 <= slot_mapping[t] < num_blocks * B (the
 * others write nothing).  DUPLICATE_SLOT: active t whose slot an earlier active token
 * has too. */
int paged_kv_check_slots(const int64_t* slot_mapping, int32_t num_tokens, const pkv_cache_desc* cache,
                         pkv_check_result* result, hipStream_t stream);

/* paged_kv_slot_mapping and paged_kv_write_positions.  SEQ_ID: token t with
 * seq_ids[t] >= num_seqs.  DUPLICATE_SLOT: as paged_kv_check_slots over the slots the
 * other tokens resolve to (by the rule of paged_kv_slot_mapping; block_tables is
 * [num_seqs][max_blocks_per_seq]). */
int paged_kv_check_positions(const int32_t* seq_ids, const int32_t* positions, int32_t num_tokens,
                             int32_t num_seqs, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const pkv_cache_desc* cache, pkv_check_result* result, hipStream_t stream);

/* paged_attention_decode, _noalloc (window = sinks = 0) and _window.  CONTEXT_LEN:
 * sequence s with context_lens[s] outside [0, max_context_len].  BLOCK_ID: for every
 * other sequence, entry j of its table row is read when block j holds an attended token
 * (any of its first context_lens[s] tokens; with window > 0, positions >=
 * context_lens[s] - window or < sinks); a read entry outside [0, num_blocks) is a
 * violation. */
int paged_attention_check_decode(int32_t num_seqs, const pkv_cache_desc* cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int32_t window, int32_t sinks,
                                 pkv_check_result* result, hipStream_t stream);

/* paged_attention_decode_shared_prefix: the decode rules (window 0), plus
 * GROUP_STARTS: entry j outside [0, num_seqs], entry 0 not 0, entry num_groups not
 * num_seqs, or (j < num_groups) group j's size group_starts[j+1] - group_starts[j]
 * negative or above max_group_size.  When group_starts breaks no rule (every sequence
 * then lies in one group, whose first sequence is f):
 * PREFIX_LEN: sequence s whose prefix_lens[s] is negative, not a multiple of B, above
 * max_prefix_len or context_lens[s], or unequal to prefix_lens[f];
 * PREFIX_BLOCKS: entry j < prefix_lens[f] / B of a sequence s != f that differs from
 * entry j of f's row (checked when prefix_lens[f] is non-negative, a multiple of B and
 * at most max_prefix_len).  Host-side errors as for the call (num_groups, bounds). */
int paged_attention_check_shared_prefix(int32_t num_seqs, const pkv_cache_desc* cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        const int32_t* group_starts, int32_t num_groups,
                                        int32_t max_group_size, const int32_t* prefix_lens,
                                        int32_t max_prefix_len, pkv_check_result* result,
                                        hipStream_t stream);

/* paged_attention_prefill: CONTEXT_LEN as for decode.  QUERY_ROWS: sequence s whose
 * n_s = cu_q[s+1] - cu_q[s] is negative, above max_q_len or above context_lens[s], and
 * s = 0 when cu_q[0] != 0.  BLOCK_ID: a sequence breaking neither rule and with n_s >= 1
 * reads entries j < ceil(context_lens[s] / B). */
int paged_attention_check_prefill(int32_t num_seqs, const int32_t* cu_q, int32_t max_q_len,
                                  const pkv_cache_desc* cache, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t max_context_len, pkv_check_result* result, hipStream_t stream);

/* paged_kv_copy_blocks (src_ids, dst_ids) and paged_kv_swap_in (src_ids NULL, dst_ids =
 * its ids).  Pair i is *active* when dst_ids[i] and (if given) src_ids[i] lie in [0,
 * num_blocks) (the others move nothing).  BLOCK_PAIR: active i whose destination an
 * earlier active pair has too, or equals the source of any active pair (itself included). */
int paged_kv_check_block_ids(const int32_t* src_ids, const int32_t* dst_ids, int32_t num,
                             const pkv_cache_desc* cache, pkv_check_result* result, hipStream_t stream);

/* ----------------------------------------------------------------- block pool ---
 * Host-side refcounted free list of one cache's physical blocks ("PagedAttention por
 * dentro...", section "El pool de bloques": one pool shared by every session).  A
 * block is free (count 0) or allocated (count >= 1).  Every call keeps free +
 * allocated == pool size; a call that fails changes nothing.  Thread-safe (one lock
 * per pool).  The pool's host memory is allocated by pkv_pool_create and freed by
 * pkv_pool_destroy; nothing on the device.
 *   pkv_pool_alloc   : n free blocks, count 1 each, into ids_out (all or nothing;
 *                      PKV_ERR_POOL_EXHAUSTED when fewer are free)
 *   pkv_pool_share   : one more reference to each (prefix caching, forked branches)
 *   pkv_pool_release : one reference less to each (an ID may repeat); a block whose
 *                      count reaches 0 is free again
 *   pkv_pool_cow     : before writing into block id: returns 0 with *id_out = id when
 *                      the caller holds the only reference, else 1 with *id_out a
 *                      fresh block (count 1) whose contents the caller copies with
 *                      paged_kv_copy_blocks, id losing the caller's reference
 * Errors: PKV_ERR_BLOCK_STATE for an ID out of range or not allocated (or released
 * more times than referenced), PKV_ERR_NULL, PKV_ERR_SHAPE for n < 0.
 */
typedef struct pkv_block_pool pkv_block_pool;
pkv_block_pool* pkv_pool_create(int32_t num_blocks); /* NULL if num_blocks <= 0 or no memory */
void pkv_pool_destroy(pkv_block_pool* pool);
int pkv_pool_alloc(pkv_block_pool* pool, int32_t n, int32_t* ids_out);
int pkv_pool_share(pkv_block_pool* pool, const int32_t* ids, int32_t n);
int pkv_pool_release(pkv_block_pool* pool, const int32_t* ids, int32_t n);
int pkv_pool_cow(pkv_block_pool* pool, int32_t id, int32_t* id_out);
int32_t pkv_pool_free_count(pkv_block_pool* pool);              /* >= 0, or an error */
int32_t pkv_pool_refcount(pkv_block_pool* pool, int32_t id);    /* >= 0, or an error */

/* Static description of a status code. */
const char* pkv_status_string(int status);

/* ABI version: bumps when any signature or layout above changes. */
int32_t pkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
