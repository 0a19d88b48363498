"""Seeded synthetic decode-step inputs: context-length mixes, block pools, values.

This module is the only code shared by the HIP path's tests/bench and by the
oracle's tests.  It holds none of the method's arithmetic: it draws random
numbers, picks context lengths and hands out physical block IDs from a pool.
Slot resolution, the cache write (including fp8 quantisation) and attention
are each implemented independently by the two sides that consume these inputs.

Shapes follow the pages' examples:
  * Llama-3-8B-style GQA, 32 query heads over 8 KV heads, d_h = 128 ("KV cache:
    la memoria de trabajo...", section "Trucos para que el cuaderno sea mas fino",
    and the per-model table under "El precio: cuanto pesa la mochila");
  * 70B-style 64 query heads over 8 KV heads ("Optimizacion de Inferencia LLM",
    section "El Cuello de Botella de Atencion...");
  * 16-token blocks by default, 32 as the large variant ("La despensa por
    casilleros", table in "El compromiso del tamano de bloque");
  * shared prefixes mapped to the same physical blocks ("La despensa por
    casilleros", section "Prefix caching: compartir casilleros con copy-on-write").

Value representation (numpy): f32 -> float32, f16 -> float16, bf16 -> uint16
(raw bits), fp8 (OCP e4m3fn) -> uint8 (raw bits).
"""
from __future__ import annotations

import dataclasses
import math
from collections import deque
from dataclasses import dataclass, field

import numpy as np
import torch

# dtype codes shared with the C ABI enum (values only; no arithmetic).
DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
NUMPY_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}
# A quiet NaN in each storage format: free pool blocks, the tails of partially
# filled blocks and the block-table padding target are filled with it, so any
# read of a byte outside the live context shows up as a NaN in the output.
POISON_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "fp8": 0x7F}


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    kv_dtype: str
    src_dtype: str  # dtype of the new K/V vectors handed to the write
    out_dtype: str
    ctx_kind: str  # "fixed" | "uniform" | "lognormal" | "prefix" | "const"
    ctx_params: tuple
    partition_size: int = 0  # 0 = library's choice, -1 = single pass, else tokens
    pool_factor: float = 1.25
    pool_blocks: int = 0  # explicit pool size (0 = ceil(pool_factor * live) + 1)
    seed: int = 0
    # "prefix" contexts: the sequences form this many contiguous groups (group k is
    # sequences [N k / groups, N (k+1) / groups)); each group shares its own prefix blocks.
    prefix_groups: int = 1
    # decode over a sliding window: the last `window` tokens of each context plus its
    # first `sinks` (0 = the whole context)
    window: int = 0
    sinks: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


# The five decode-layer workloads.  Seeds are fixed per workload.
TINY = DecodeConfig("tiny-fp32-4seq", 4, 4, 2, 64, 16, "f32", "f32", "f32", "f32",
                    "fixed", (7, 16, 33, 100), pool_blocks=32, seed=1001)
LLAMA8B = DecodeConfig("llama3-8b-shaped-bf16-64seq", 64, 32, 8, 128, 16, "bf16", "bf16",
                       "bf16", "bf16", "uniform", (128, 4096), seed=1002)
R70B_FP8 = DecodeConfig("70b-shaped-fp8kv-128seq", 128, 64, 8, 128, 16, "bf16", "fp8",
                        "bf16", "bf16", "lognormal", (1024, 1.0, 16, 8192), seed=1003)
PREFIX = DecodeConfig("prefix-sharing-bf16-256seq-b32", 256, 32, 8, 128, 32, "bf16", "bf16",
                      "bf16", "bf16", "prefix", (2048, 0, 512), seed=1004)
LONGCTX = DecodeConfig("long-context-bf16-8seq-32k", 8, 32, 8, 128, 16, "bf16", "bf16",
                       "bf16", "bf16", "const", (32768,), partition_size=512, seed=1005)
CONFIGS = [TINY, LLAMA8B, R70B_FP8, PREFIX, LONGCTX]
# Beyond the five: the long-context layer decoded over a Mistral-style window of the last
# 4096 tokens plus 4 attention-sink tokens (the blocks in between freed).
LONGCTX_WINDOW = LONGCTX.replace(name="long-context-window4096-sinks4-bf16-8seq-32k", window=4096,
                                 sinks=4, partition_size=0)
EXTRA_CONFIGS = [LONGCTX_WINDOW]


def context_lengths(cfg: DecodeConfig, rng: np.random.Generator) -> np.ndarray:
    """Context length per sequence, counting the new token (it sits at ctx-1)."""
    n = cfg.num_seqs
    k, p = cfg.ctx_kind, cfg.ctx_params
    if k == "fixed":
        out = np.asarray(p, dtype=np.int64)
        assert out.size == n
    elif k == "uniform":
        out = rng.integers(p[0], p[1] + 1, size=n)
    elif k == "lognormal":
        median, sigma, lo, hi = p
        out = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=n))), lo, hi)
    elif k == "prefix":
        prefix, lo, hi = p
        out = prefix + rng.integers(lo, hi + 1, size=n) + 1
    elif k == "const":
        out = np.full(n, p[0])
    else:
        raise ValueError(k)
    return out.astype(np.int32)


class BlockPool:
    """Host-side pool of physical block IDs with reference counts.

    The pool is sized once; free IDs come out of a seeded permutation so that a
    sequence's logical blocks land anywhere in the cache ("La despensa por
    casilleros", section "El block manager: el bibliotecario de la despensa";
    "PagedAttention por dentro", section "El pool de bloques").
    """

    def __init__(self, num_blocks: int, rng: np.random.Generator):
        self.num_blocks = int(num_blocks)
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)
        self._free = deque(int(b) for b in rng.permutation(self.num_blocks))

    def allocate(self) -> int:
        if not self._free:
            raise RuntimeError("block pool exhausted")
        b = self._free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def share(self, block: int) -> int:
        assert self.refcount[block] > 0, "sharing a free block"
        self.refcount[block] += 1
        return block

    def release(self, block: int) -> None:
        assert self.refcount[block] > 0, "double free"
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            self._free.append(block)

    @property
    def num_free(self) -> int:
        return len(self._free)

    @property
    def num_allocated(self) -> int:
        return int((self.refcount > 0).sum())

    def free_ids(self) -> list[int]:
        return list(self._free)


@dataclass
class Workload:
    cfg: DecodeConfig
    seed: int
    context_lens: np.ndarray  # int32 [N]
    block_tables: np.ndarray  # int32 [N][max_blocks]
    num_blocks: int
    sentinel_block: int  # every padding entry of block_tables points here
    refcount: np.ndarray  # int32 [num_blocks]
    free_blocks: list
    hist_seq: np.ndarray  # int32 [T_hist]: tokens already in the cache, written in bulk
    hist_pos: np.ndarray  # int32 [T_hist]
    hist_k: np.ndarray  # [T_hist][H_kv][D] in src_dtype storage
    hist_v: np.ndarray
    new_k: np.ndarray  # [N][H_kv][D]: the step's new token per sequence
    new_v: np.ndarray
    q: np.ndarray  # [N][H_q][D] in q_dtype storage
    k_scale: float
    v_scale: float
    scale: float
    shared_blocks: list = field(default_factory=list)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def new_seq(self) -> np.ndarray:
        return np.arange(self.cfg.num_seqs, dtype=np.int32)

    @property
    def new_pos(self) -> np.ndarray:
        return (self.context_lens - 1).astype(np.int32)

    def prefix_group_starts(self) -> np.ndarray:
        """First sequence of each prefix-sharing group, then num_seqs (int32)."""
        n = self.cfg.num_seqs
        k = self.cfg.prefix_groups if self.cfg.ctx_kind == "prefix" else 1
        return np.array([n * i // k for i in range(k + 1)], dtype=np.int32)

    def prefix_owner(self, s: int) -> int:
        """The sequence whose cached rows hold s's shared prefix (its group's first)."""
        starts = self.prefix_group_starts()
        return int(starts[np.searchsorted(starts, s, side="right") - 1])

    def logical_kv(self, s: int):
        """K and V of sequence s in logical token order (src storage), new token last."""
        ctx = int(self.context_lens[s])
        pos_to_row = {}
        prefix = self._shared_prefix_len()
        for row in np.nonzero(self.hist_seq == s)[0]:
            pos_to_row[int(self.hist_pos[row])] = int(row)
        owner = self.prefix_owner(s) if prefix else s
        if prefix and s != owner:
            for row in np.nonzero((self.hist_seq == owner) & (self.hist_pos < prefix))[0]:
                pos_to_row[int(self.hist_pos[row])] = int(row)
        rows = [pos_to_row[p] for p in range(ctx - 1)]
        k = np.concatenate([self.hist_k[rows], self.new_k[s:s + 1]], axis=0)
        v = np.concatenate([self.hist_v[rows], self.new_v[s:s + 1]], axis=0)
        return k, v

    def _shared_prefix_len(self) -> int:
        return int(self.cfg.ctx_params[0]) if self.cfg.ctx_kind == "prefix" else 0

    def kv_bytes_algorithmic(self) -> int:
        """Bytes of K and V one decode pass must read, each sequence's whole context."""
        c = self.cfg
        return int(self.context_lens.astype(np.int64).sum()) * c.num_kv_heads * c.head_dim * 2 * DTYPE_BYTES[c.kv_dtype]

    def kv_bytes_unique(self) -> int:
        """Distinct K and V bytes one decode pass reads (shared prefix counted once)."""
        c = self.cfg
        prefix = self._shared_prefix_len()
        tokens = int(self.context_lens.astype(np.int64).sum())
        if prefix:
            groups = len(self.prefix_group_starts()) - 1
            tokens -= prefix * (c.num_seqs - groups)
        return tokens * c.num_kv_heads * c.head_dim * 2 * DTYPE_BYTES[c.kv_dtype]


def _random_values(gen: torch.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) fp32 draws cast (round-to-nearest-even) to the storage dtype.

    Values are drawn in fixed chunks so the stream does not depend on memory.
    """
    total = int(np.prod(shape))
    out = np.empty(total, dtype=NUMPY_STORAGE[dtype])
    chunk = 1 << 24
    for start in range(0, total, chunk):
        n = min(chunk, total - start)
        x = torch.randn(n, generator=gen, dtype=torch.float32)
        if dtype == "f32":
            out[start:start + n] = x.numpy()
        elif dtype == "f16":
            out[start:start + n] = x.to(torch.float16).numpy()
        elif dtype == "bf16":
            out[start:start + n] = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        else:
            raise ValueError(f"values are not drawn directly in {dtype}")
    return out.reshape(shape)


def _abs_max_as_f32(x: np.ndarray, dtype: str) -> np.float32:
    if dtype == "bf16":
        f = (x.astype(np.uint32) << 16).view(np.float32)
    else:
        f = x.astype(np.float32)
    return np.float32(np.abs(f).max()) if f.size else np.float32(0)


def make_workload(cfg: DecodeConfig, seed: int | None = None,
                  context_lens: np.ndarray | None = None) -> Workload:
    """Build one decode step's inputs for `cfg` (context lens may be overridden)."""
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)
    N, Hkv, D, B = cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim, cfg.block_size

    ctx = context_lengths(cfg, rng) if context_lens is None else np.asarray(context_lens, np.int32)
    assert ctx.shape == (N,)
    nblk = (ctx.astype(np.int64) + B - 1) // B
    prefix = int(cfg.ctx_params[0]) if cfg.ctx_kind == "prefix" else 0
    assert prefix % B == 0, "a shared prefix must end on a block boundary"
    shared_n = prefix // B
    ngroups = cfg.prefix_groups if prefix else 1
    starts = [N * i // ngroups for i in range(ngroups + 1)]
    first = set(starts[:-1])  # the first sequence of each group owns its prefix rows
    live = int(nblk.sum()) - shared_n * max(N - ngroups, 0)
    num_blocks = cfg.pool_blocks or int(math.ceil(cfg.pool_factor * live)) + 1
    assert num_blocks >= live + 1, "pool too small for the live blocks plus the sentinel"

    pool = BlockPool(num_blocks, rng)
    max_blocks = max(int(nblk.max()) if N else 1, 1)
    tables = np.empty((N, max_blocks), dtype=np.int32)
    shared = [pool.allocate() for _ in range(shared_n)]  # group 0's prefix blocks
    all_shared = list(shared)
    for s in range(N):
        if s in first and s > 0:  # a later group: its own prefix blocks
            shared = [pool.allocate() for _ in range(shared_n)]
            all_shared += shared
        ids = []
        for j in range(int(nblk[s])):
            ids.append(pool.share(shared[j]) if j < shared_n and s not in first else
                       (shared[j] if j < shared_n else pool.allocate()))
        tables[s, :len(ids)] = ids
        tables[s, len(ids):] = -2  # filled below with the sentinel
    sentinel = pool.allocate()
    tables[tables == -2] = sentinel

    # Cached history: every position before the new token; each shared prefix once.
    seqs, poss = [], []
    for s in range(N):
        start = prefix if (prefix and s not in first) else 0
        n_hist = int(ctx[s]) - 1 - start
        if n_hist > 0:
            seqs.append(np.full(n_hist, s, np.int32))
            poss.append(np.arange(start, start + n_hist, dtype=np.int32))
    hist_seq = np.concatenate(seqs) if seqs else np.zeros(0, np.int32)
    hist_pos = np.concatenate(poss) if poss else np.zeros(0, np.int32)
    T = hist_seq.size

    src = cfg.src_dtype
    q = _random_values(gen, (N, cfg.num_q_heads, D), cfg.q_dtype)
    new_k = _random_values(gen, (N, Hkv, D), src)
    new_v = _random_values(gen, (N, Hkv, D), src)
    hist_k = _random_values(gen, (T, Hkv, D), src)
    hist_v = _random_values(gen, (T, Hkv, D), src)

    k_scale = v_scale = 1.0
    if cfg.kv_dtype == "fp8":
        # Per-tensor scale: the largest magnitude maps to the largest finite e4m3 value.
        e4m3_max = np.float32(448.0)
        k_scale = float(max(_abs_max_as_f32(hist_k, src), _abs_max_as_f32(new_k, src)) / e4m3_max)
        v_scale = float(max(_abs_max_as_f32(hist_v, src), _abs_max_as_f32(new_v, src)) / e4m3_max)

    return Workload(cfg=cfg, seed=seed, context_lens=ctx, block_tables=tables,
                    num_blocks=num_blocks, sentinel_block=sentinel,
                    refcount=pool.refcount.copy(), free_blocks=pool.free_ids(),
                    hist_seq=hist_seq, hist_pos=hist_pos, hist_k=hist_k, hist_v=hist_v,
                    new_k=new_k, new_v=new_v, q=q, k_scale=k_scale, v_scale=v_scale,
                    scale=float(np.float32(1.0 / math.sqrt(D))), shared_blocks=all_shared)


def cache_shape(w: Workload) -> tuple:
    c = w.cfg
    return (w.num_blocks, c.num_kv_heads, c.block_size, c.head_dim)


def prefill_queries(w: Workload, chunk_lens, seed: int = 77):
    """Query rows of a chunked-prefill step over workload w: sequence s brings
    chunk_lens[s] query tokens (the last ones of its context, <= its length), drawn
    ~N(0,1) in the query dtype like decode queries.  Returns (q [rows][H_q][d_h],
    cu_q [N + 1] int32)."""
    c = w.cfg
    n = np.asarray(chunk_lens, dtype=np.int32)
    assert n.shape == (c.num_seqs,) and (n >= 0).all() and (n <= w.context_lens).all()
    cu = np.zeros(c.num_seqs + 1, np.int32)
    cu[1:] = np.cumsum(n)
    gen = torch.Generator().manual_seed(seed)
    q = _random_values(gen, (int(cu[-1]), c.num_q_heads, c.head_dim), c.q_dtype)
    return q, cu


def poisoned_cache(w: Workload) -> np.ndarray:
    """A cache array of the workload's KV dtype with every element set to NaN."""
    dt = w.cfg.kv_dtype
    storage = NUMPY_STORAGE[dt]
    bits = POISON_BITS[dt]
    if dt == "f32":
        return np.full(cache_shape(w), bits, dtype=np.uint32).view(np.float32)
    if dt == "f16":
        return np.full(cache_shape(w), bits, dtype=np.uint16).view(np.float16)
    return np.full(cache_shape(w), bits, dtype=storage)
