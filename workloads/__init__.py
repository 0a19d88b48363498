"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle's tests."""
from .synth import (CONFIGS, DTYPE_BYTES, DTYPE_CODES, EXTRA_CONFIGS, LLAMA8B, LONGCTX,
                    LONGCTX_WINDOW, NUMPY_STORAGE,
                    POISON_BITS, PREFIX, R70B_FP8, TINY, BlockPool, DecodeConfig, Workload,
                    cache_shape, context_lengths, make_workload, poisoned_cache, prefill_queries)
