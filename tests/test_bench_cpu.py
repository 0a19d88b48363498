"""bench.py's bookkeeping on the CPU: the algorithmic bytes its roofline figures divide by,
against the closed form and the figures of the pages' workloads, and its one-GPU refusal.

Algorithmic bytes of one decode call: each sequence's K and V once per KV head
(ctx * H_kv * d_h * 2 * bytes per element), its query and output rows, its block-table
entries and context length ("Capitulo 2 -- KV cache...", section "Una formula util para
estimar memoria de KV": M_KV = T * L * 2 * H_kv * d_h * b, per layer; the paged reads of
"PagedAttention por dentro...", section "El kernel CUDA").  A shared prefix counts once per
group of sequences mapping the same physical blocks when priced against HBM ("La despensa
por casilleros", section "Prefix caching: compartir casilleros con copy-on-write").
"""
import subprocess
import sys
import types
from pathlib import Path

import numpy as np

import bench
from workloads import CONFIGS, LLAMA8B, PREFIX, TINY, make_workload
from workloads.synth import context_lengths

ROOT = Path(__file__).resolve().parents[1]
ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}


def _stand_in(cfg):
    """The fields algorithmic_bytes reads, with the configuration's own context lengths
    (no K/V drawn: the full-size caches would take gigabytes)."""
    ctx = context_lengths(cfg, np.random.default_rng(cfg.seed))
    kv = int(ctx.astype(np.int64).sum()) * cfg.num_kv_heads * cfg.head_dim * 2 * ELEM[cfg.kv_dtype]
    return types.SimpleNamespace(cfg=cfg, context_lens=ctx, kv_bytes_unique=lambda: kv, shared_blocks=[])


def test_tiny_workload_bytes():
    """Contexts {7, 16, 33, 100}, 2 KV heads of 64 fp32 dims: 156 tokens x 1024 bytes of K
    and V, 12 table entries + 4 context lengths, 4 x 4 query and output rows of 256 bytes."""
    w = make_workload(TINY)
    b = bench.algorithmic_bytes(w)
    assert b["kv"] == 159_744
    assert b["decode"] == 159_744 + (12 + 4) * 4 + 2 * 4 * 4 * 64 * 4 == 168_000
    assert bench.roofline_bytes(b, w) == b["decode"]


def test_full_size_closed_forms():
    """The five workloads at full size: bytes per token (4 KiB for 8 bf16 KV heads of 128
    dims, 2 KiB in fp8), the 32K layer's 1 GiB, and the query/output bytes."""
    per_token = {1: 1024, 2: 4096, 3: 2048, 4: 4096, 5: 4096}
    qo = {1: 8192, 2: 1 << 20, 3: 4 << 20, 4: 4 << 20, 5: 128 << 10}
    for i, cfg in enumerate(CONFIGS, start=1):
        w = _stand_in(cfg)
        b = bench.algorithmic_bytes(w)
        ctx = w.context_lens.astype(np.int64)
        assert b["kv"] == int(ctx.sum()) * per_token[i], cfg.name
        table = int(((ctx + cfg.block_size - 1) // cfg.block_size).sum()) * 4 + 4 * cfg.num_seqs
        assert b["decode"] == b["kv"] + table + qo[i], cfg.name
    assert bench.algorithmic_bytes(_stand_in(CONFIGS[4]))["kv"] == 1 << 30


def test_shared_prefix_priced_once_per_group():
    """Sequences of a group map one prefix's physical blocks: the roofline bytes count it
    once per group, the logical bytes once per sequence."""
    cfg = PREFIX.replace(num_seqs=6, prefix_groups=2, ctx_params=(64, 0, 40))
    w = make_workload(cfg)
    b = bench.algorithmic_bytes(w)
    per_token = cfg.num_kv_heads * cfg.head_dim * 2 * 2
    assert b["kv_unique"] == b["kv"] - (6 - 2) * 64 * per_token
    assert bench.roofline_bytes(b, w) == b["decode_unique"] == b["decode"] - (6 - 2) * 64 * per_token
    plain = make_workload(LLAMA8B.replace(num_seqs=3, ctx_kind="fixed", ctx_params=(5, 40, 300)))
    pb = bench.algorithmic_bytes(plain)
    assert pb["kv_unique"] == pb["kv"] and bench.roofline_bytes(pb, plain) == pb["decode"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
