"""ctypes binding of the library's input checks (the paged_*_check_* calls of
include/pagedkv.h): argument marshalling only.  Each function allocates the 24-byte
device result, runs the check on the given stream, waits for it and returns a
CheckResult; the rules themselves run in the library's kernels.

Debug mode: with PAGEDKV_DEBUG set (to anything but 0), the binding's entry points run
the matching check before their call and raise PreconditionError instead of launching
it when an entry breaks a rule.  The check waits for the stream, so debug mode is not
for code under graph capture.
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple

import numpy as np
import torch

from ._binding import CacheDesc, _check, _ptr, _stream, cache_desc, load_library

CHECK_CODES = {0: "ok", 1: "duplicate slot", 2: "sequence ID", 3: "context length", 4: "block ID",
               5: "group starts", 6: "prefix length", 7: "prefix blocks", 8: "query rows", 9: "block pair"}
RESULT_BYTES = 24


class CheckResult(NamedTuple):
    violations: int
    code: int   # the lowest code violated (0: none)
    index: int  # the lowest index violating it (-1: none)

    @property
    def what(self) -> str:
        return CHECK_CODES.get(self.code, str(self.code))


class PreconditionError(RuntimeError):
    def __init__(self, fn: str, result: CheckResult):
        super().__init__(f"{fn}: {result.violations} input entries break its preconditions; first: "
                         f"{result.what} at index {result.index}")
        self.result = result


_declared = False


def _lib():
    global _declared
    lib = load_library()
    if not _declared:
        vp, i32, desc, cint = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(CacheDesc), ctypes.c_int
        sig = {
            "paged_kv_check_slots": [vp, i32, desc, vp, vp],
            "paged_kv_check_positions": [vp, vp, i32, i32, vp, i32, desc, vp, vp],
            "paged_attention_check_decode": [i32, desc, vp, i32, vp, i32, i32, i32, vp, vp],
            "paged_attention_check_shared_prefix": [i32, desc, vp, i32, vp, i32, vp, i32, i32, vp, i32, vp, vp],
            "paged_attention_check_prefill": [i32, vp, i32, desc, vp, i32, vp, i32, vp, vp],
            "paged_kv_check_block_ids": [vp, vp, i32, desc, vp, vp],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = cint
        _declared = True
    return lib


def _run(name: str, device, stream, call) -> CheckResult:
    result = torch.empty(RESULT_BYTES, dtype=torch.uint8, device=device)
    _check(name, call(_ptr(result), _stream(stream)))
    torch.cuda.synchronize(device)
    raw = result.cpu().numpy()
    code = int(raw[0:4].view(np.int32)[0])
    index = int(raw[8:16].view(np.int64)[0])
    violations = int(raw[16:24].view(np.int64)[0])
    return CheckResult(violations, code, index)


def _i32(t: torch.Tensor) -> torch.Tensor:
    assert t.dtype == torch.int32, t.dtype
    return t


def paged_kv_check_slots(slot_mapping: torch.Tensor, k_cache: torch.Tensor, kv_dtype=None,
                         stream=None) -> CheckResult:
    """Duplicate slots among those paged_kv_write would write."""
    assert slot_mapping.dtype == torch.int64
    desc = cache_desc(k_cache, kv_dtype)
    return _run("paged_kv_check_slots", k_cache.device, stream, lambda r, s: _lib().paged_kv_check_slots(
        _ptr(slot_mapping), slot_mapping.numel(), ctypes.byref(desc), r, s))


def paged_kv_check_positions(seq_ids: torch.Tensor, positions: torch.Tensor, block_tables: torch.Tensor,
                             k_cache: torch.Tensor, kv_dtype=None, stream=None) -> CheckResult:
    """Sequence IDs past the table and duplicate resolved slots (paged_kv_write_positions)."""
    assert seq_ids.numel() == positions.numel()
    desc = cache_desc(k_cache, kv_dtype)
    return _run("paged_kv_check_positions", k_cache.device, stream, lambda r, s: _lib().paged_kv_check_positions(
        _ptr(_i32(seq_ids)), _ptr(_i32(positions)), seq_ids.numel(), block_tables.shape[0],
        _ptr(_i32(block_tables)), block_tables.shape[1], ctypes.byref(desc), r, s))


def paged_attention_check_decode(block_tables: torch.Tensor, context_lens: torch.Tensor, max_context_len: int,
                                 k_cache: torch.Tensor, window: int = 0, sinks: int = 0, kv_dtype=None,
                                 stream=None) -> CheckResult:
    """Context lengths and the block IDs a decode (window 0) or windowed decode reads."""
    desc = cache_desc(k_cache, kv_dtype)
    return _run("paged_attention_check_decode", k_cache.device, stream,
                lambda r, s: _lib().paged_attention_check_decode(
                    context_lens.numel(), ctypes.byref(desc), _ptr(_i32(block_tables)), block_tables.shape[1],
                    _ptr(_i32(context_lens)), int(max_context_len), int(window), int(sinks), r, s))


def paged_attention_check_shared_prefix(block_tables: torch.Tensor, context_lens: torch.Tensor,
                                        max_context_len: int, group_starts: torch.Tensor,
                                        prefix_lens: torch.Tensor, max_group_size: int, max_prefix_len: int,
                                        k_cache: torch.Tensor, kv_dtype=None, stream=None) -> CheckResult:
    """The decode rules plus the grouping, prefix lengths and shared prefix entries."""
    desc = cache_desc(k_cache, kv_dtype)
    return _run("paged_attention_check_shared_prefix", k_cache.device, stream,
                lambda r, s: _lib().paged_attention_check_shared_prefix(
                    context_lens.numel(), ctypes.byref(desc), _ptr(_i32(block_tables)), block_tables.shape[1],
                    _ptr(_i32(context_lens)), int(max_context_len), _ptr(_i32(group_starts)),
                    group_starts.numel() - 1, int(max_group_size), _ptr(_i32(prefix_lens)),
                    int(max_prefix_len), r, s))


def paged_attention_check_prefill(cu_q: torch.Tensor, max_q_len: int, block_tables: torch.Tensor,
                                  context_lens: torch.Tensor, max_context_len: int, k_cache: torch.Tensor,
                                  kv_dtype=None, stream=None) -> CheckResult:
    """Context lengths, query rows and the block IDs a chunked prefill reads."""
    desc = cache_desc(k_cache, kv_dtype)
    return _run("paged_attention_check_prefill", k_cache.device, stream,
                lambda r, s: _lib().paged_attention_check_prefill(
                    context_lens.numel(), _ptr(_i32(cu_q)), int(max_q_len), ctypes.byref(desc),
                    _ptr(_i32(block_tables)), block_tables.shape[1], _ptr(_i32(context_lens)),
                    int(max_context_len), r, s))


def paged_kv_check_block_ids(src_ids: torch.Tensor | None, dst_ids: torch.Tensor, k_cache: torch.Tensor,
                             kv_dtype=None, stream=None) -> CheckResult:
    """Destinations of a copy-on-write (src_ids given) or a swap in (src_ids None)."""
    if src_ids is not None:
        assert src_ids.numel() == dst_ids.numel()
    desc = cache_desc(k_cache, kv_dtype)
    return _run("paged_kv_check_block_ids", k_cache.device, stream, lambda r, s: _lib().paged_kv_check_block_ids(
        _ptr(_i32(src_ids)) if src_ids is not None else None, _ptr(_i32(dst_ids)), dst_ids.numel(),
        ctypes.byref(desc), r, s))


def debug_enabled() -> bool:
    return os.environ.get("PAGEDKV_DEBUG", "") not in ("", "0")


def raise_if_broken(fn: str, result: CheckResult) -> None:
    if result.violations:
        raise PreconditionError(fn, result)
