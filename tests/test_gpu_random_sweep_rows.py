"""Seeded random sweeps of the many-row attention entry points -- shared-prefix decode
and chunked prefill -- through the C ABI (GPU only), each case against the oracle.

Shared-prefix cases draw the cache dtype (bf16, f16, fp8 e4m3fn with bf16 or f16
queries), head dim, block size, KV heads, group size, 1-40 sequences in 1-4 groups that
share prefix blocks of 1-12 blocks, suffixes of 0-200 tokens, and the grouping declared
to the entry point: the true one, a shorter declared prefix, or singleton groups.  The
result must be what plain decode computes: the oracle's decode, within the decode bar.

Prefill cases draw the same dtypes and shapes, 1-4 sequences of 1-500 tokens and each
one's chunk (the last 1-160 tokens of its context, a single token or the whole prompt
among them): every output against the oracle's causal attention, within the same bar.
The draw is printed before each case runs.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, out_to_f64, to_device, torch_dtype
from helpers import oracle_step
from workloads import LLAMA8B, PREFIX, make_workload, prefill_queries

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))
N_PREFIX_CASES = 60
N_PREFILL_CASES = 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _dtypes(rng):
    kv = ["bf16", "f16", "fp8"][int(rng.integers(3))]
    q = {"bf16": "bf16", "f16": "f16", "fp8": ["bf16", "f16"][int(rng.integers(2))]}[kv]
    out = q if rng.random() < 0.7 else "f32"
    return kv, q, out


def _prefix_draw(i: int):
    rng = np.random.default_rng(9000 + i)
    kv, q, out = _dtypes(rng)
    D, B = int(rng.choice([64, 128])), int(rng.choice([16, 32]))
    hkv, G = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 3, 4, 8, 16]))
    n = int(rng.integers(1, 41))
    groups = int(rng.integers(1, min(4, n) + 1))
    prefix = B * int(rng.integers(1, 13))
    cfg = PREFIX.replace(name=f"prefix-sweep-{i:03d}", num_seqs=n, num_q_heads=G * hkv, num_kv_heads=hkv,
                         head_dim=D, block_size=B, q_dtype=q, kv_dtype=kv, src_dtype=q, out_dtype=out,
                         ctx_params=(prefix, 0, int(rng.integers(0, 201))), prefix_groups=groups,
                         seed=9000 + i)
    mode = ["true", "true", "shorter", "singletons"][int(rng.integers(4))]
    cut = B * int(rng.integers(1, prefix // B + 1))  # declared prefix shorter by this much
    return cfg, mode, cut


@pytest.mark.parametrize("i", range(N_PREFIX_CASES), ids=[f"case{i:03d}" for i in range(N_PREFIX_CASES)])
def test_shared_prefix_sweep(orc, i):
    cfg, mode, cut = _prefix_draw(i)
    w = make_workload(cfg)
    n, prefix = cfg.num_seqs, int(cfg.ctx_params[0])
    if mode == "singletons":  # every sequence its own group, with the full shared prefix
        starts, pl = np.arange(n + 1, dtype=np.int32), np.full(n, prefix, np.int32)
    else:
        starts = np.asarray(w.prefix_group_starts(), np.int32)
        pl = np.full(n, prefix - (cut if mode == "shorter" else 0), np.int32)
    print(f"shared-prefix sweep case {i}: kv={cfg.kv_dtype} q={cfg.q_dtype} out={cfg.out_dtype} "
          f"D={cfg.head_dim} B={cfg.block_size} Hkv={cfg.num_kv_heads} G={cfg.group} N={n} "
          f"groups={list(starts)} declared prefix={int(pl.max())} of {prefix}", flush=True)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    pkv.paged_attention_decode_shared_prefix(
        g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale, g.out, w.max_context_len,
        torch.from_numpy(starts).cuda(), torch.from_numpy(pl).cuda(), int(np.diff(starts).max()),
        int(pl.max()), kv_dtype=g.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    got = out_to_f64(g.out)
    _, _, _, ref = oracle_step(orc, w, threads=THREADS)
    assert_close_to_oracle(got, ref, cfg.kv_dtype, f"shared-prefix sweep case {i}")


def _prefill_draw(i: int):
    rng = np.random.default_rng(11000 + i)
    kv, q, out = _dtypes(rng)
    D, B = int(rng.choice([64, 128])), int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 3, 4, 8, 16) if g * hkv <= 32]))
    n = int(rng.integers(1, 5))
    ctx = rng.integers(1, 501, n)
    pick = rng.random(n)
    chunk = np.where(pick < 0.15, 1, np.where(pick < 0.3, np.minimum(ctx, 160),
                                              rng.integers(1, np.minimum(ctx, 160) + 1)))
    cfg = LLAMA8B.replace(name=f"prefill-sweep-{i:03d}", num_seqs=n, num_q_heads=G * hkv, num_kv_heads=hkv,
                          head_dim=D, block_size=B, q_dtype=q, kv_dtype=kv, src_dtype=q, out_dtype=out,
                          ctx_kind="fixed", ctx_params=tuple(int(x) for x in ctx), seed=11000 + i)
    return cfg, tuple(int(x) for x in chunk)


@pytest.mark.parametrize("i", range(N_PREFILL_CASES), ids=[f"case{i:03d}" for i in range(N_PREFILL_CASES)])
def test_prefill_sweep(orc, i):
    cfg, chunks = _prefill_draw(i)
    print(f"prefill sweep case {i}: kv={cfg.kv_dtype} q={cfg.q_dtype} out={cfg.out_dtype} D={cfg.head_dim} "
          f"B={cfg.block_size} Hkv={cfg.num_kv_heads} G={cfg.group} ctx={cfg.ctx_params} chunks={chunks}",
          flush=True)
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    c = w.cfg
    q, cu = prefill_queries(w, chunks, 5 + i)
    out = torch.empty((int(cu[-1]), c.num_q_heads, c.head_dim), dtype=torch_dtype(c.out_dtype), device="cuda")
    pkv.paged_attention_prefill(to_device(q, c.q_dtype), torch.from_numpy(cu).cuda(), int(max(chunks)),
                                g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale, out,
                                w.max_context_len, kv_dtype=g.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    del g
    kc, vc, _, _ = oracle_step(orc, w, pairs=np.zeros((0, 2), np.int32))
    ref = orc.prefill(q, c.q_dtype, cu, kc, vc, c.kv_dtype, w.block_tables, w.context_lens, w.scale,
                      w.k_scale, w.v_scale, threads=THREADS)
    assert_close_to_oracle(got, ref, c.kv_dtype, f"prefill sweep case {i}")
