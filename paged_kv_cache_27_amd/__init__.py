"""Paged KV cache decode path for AMD MI355X (gfx950).

The compute runs in libpagedkv.so (hand-written HIP kernels behind the C ABI
declared in include/pagedkv.h); this package only marshals torch tensors to it.
"""
from ._binding import (BF16, BlockPoolHandle, paged_attention_prefill, paged_kv_copy_blocks, paged_kv_swap_in, paged_kv_swap_out, CACHE_SHARED_BLOCKS, F16, F32, FP8_E4M3, CacheDesc, PagedKVError, cache_desc,
                       load_library, paged_attention_schedule, paged_attention_decode,
                       paged_attention_decode_noalloc, NOALLOC_SCRATCH_BYTES,
                       paged_attention_decode_window,
                       paged_attention_workspace_size, paged_kv_slot_mapping, paged_kv_write,
                       paged_kv_write_positions,
                       paged_attention_decode_shared_prefix,
                       paged_attention_shared_prefix_workspace_size,
                       pkv_abi_version, pkv_status_string, WORKSPACE_HEADER_BYTES)
from ._checks import (CHECK_CODES, CheckResult, PreconditionError, paged_attention_check_decode,
                      paged_attention_check_prefill, paged_attention_check_shared_prefix,
                      paged_kv_check_block_ids, paged_kv_check_positions, paged_kv_check_slots)

__all__ = ["BF16", "BlockPoolHandle", "paged_attention_prefill", "paged_kv_copy_blocks", "paged_kv_swap_in", "paged_kv_swap_out", "CACHE_SHARED_BLOCKS", "F16", "F32", "FP8_E4M3", "CacheDesc", "PagedKVError", "cache_desc",
           "load_library", "paged_attention_schedule", "paged_attention_decode", "paged_attention_decode_noalloc",
           "NOALLOC_SCRATCH_BYTES", "paged_attention_decode_window",
           "paged_attention_workspace_size", "paged_kv_slot_mapping", "paged_kv_write", "paged_kv_write_positions",
           "paged_attention_decode_shared_prefix", "paged_attention_shared_prefix_workspace_size",
           "pkv_abi_version", "pkv_status_string", "WORKSPACE_HEADER_BYTES",
           "CHECK_CODES", "CheckResult", "PreconditionError", "paged_attention_check_decode",
           "paged_attention_check_prefill", "paged_attention_check_shared_prefix", "paged_kv_check_block_ids",
           "paged_kv_check_positions", "paged_kv_check_slots"]
