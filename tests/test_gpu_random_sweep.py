"""Seeded random sweep of decode shapes, dtypes, context mixes and schedules, through the
C ABI (GPU only), each case against the oracle.

Each case draws, from its own seed: the cache dtype (bf16, f16, fp8 e4m3fn with bf16 or
f16 queries, f32), the output dtype, head dim 64 or 128, block size 16 or 32, 1-8 KV heads
and 1-16 query heads per KV head, 1-24 sequences whose context lengths mix empty, short,
block-edge and long ones (or groups sharing prefix blocks), the schedule (balanced, one
pass, fixed partitions of 1-16 blocks) and, for some, a sliding window with sinks whose
freed blocks point at the NaN sentinel.  The write is compared byte for byte with the
oracle's cache; every decode output within the decode bar (4e-3, fp8 KV 2e-2, times
max(1, |ref|)).  The draw is printed before each case runs.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, cache_bytes, out_to_f64
from helpers import free_blocks_outside_window, oracle_step
from workloads import LLAMA8B, make_workload

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))
N_CASES = 160


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _draw(i: int):
    """The configuration, partition request and (window, sinks) of case i."""
    rng = np.random.default_rng(7000 + i)
    kv = ["bf16", "f16", "fp8", "f32"][int(rng.integers(4))]
    q = {"bf16": "bf16", "f16": "f16", "f32": "f32", "fp8": ["bf16", "f16"][int(rng.integers(2))]}[kv]
    out = q if rng.random() < 0.7 else "f32"
    D = int(rng.choice([64, 128]))
    B = int(rng.choice([16, 32]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16] if kv != "f32" else [1, 2, 3, 4]))
    n = int(rng.integers(1, 25))
    if rng.random() < 0.2:  # groups of sequences sharing prefix blocks
        prefix = B * int(rng.integers(1, 9))
        kind, params = "prefix", (prefix, 0, int(rng.integers(1, 200)))
        groups = int(rng.integers(1, min(3, n) + 1))
    else:
        pick = rng.random(n)
        lens = np.where(pick < 0.1, 0,
                        np.where(pick < 0.35, rng.integers(1, 40, n),
                                 np.where(pick < 0.5, B * rng.integers(1, 9, n) + rng.integers(-1, 2, n),
                                          np.where(pick < 0.9, rng.integers(40, 700, n),
                                                   rng.integers(700, 2500, n)))))
        kind, params, groups = "fixed", tuple(int(max(0, x)) for x in lens), 1
    cfg = LLAMA8B.replace(name=f"sweep-{i:03d}", num_seqs=n, num_q_heads=G * hkv, num_kv_heads=hkv,
                          head_dim=D, block_size=B, q_dtype=q, kv_dtype=kv, src_dtype=q, out_dtype=out,
                          ctx_kind=kind, ctx_params=params, prefix_groups=groups, seed=7000 + i)
    part = [0, 0, -1, B, 2 * B, 4 * B, 16 * B][int(rng.integers(7))]
    window = sinks = 0
    if kind == "fixed" and rng.random() < 0.3:
        window = int(rng.integers(1, 300))
        sinks = int(rng.choice([0, 1, 4, 17]))
    return cfg, part, window, sinks


@pytest.mark.parametrize("i", range(N_CASES), ids=[f"case{i:03d}" for i in range(N_CASES)])
def test_random_sweep(orc, i):
    cfg, part, window, sinks = _draw(i)
    print(f"sweep case {i}: kv={cfg.kv_dtype} q={cfg.q_dtype} out={cfg.out_dtype} D={cfg.head_dim} "
          f"B={cfg.block_size} Hkv={cfg.num_kv_heads} G={cfg.group} N={cfg.num_seqs} ctx={cfg.ctx_kind} "
          f"partition={part} window={window} sinks={sinks}", flush=True)
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    torch.cuda.synchronize()
    kc, vc, ns, ref = oracle_step(orc, w, threads=THREADS)
    assert np.array_equal(g.new_slots.cpu().numpy(), ns)
    assert np.array_equal(cache_bytes(g.k_cache).reshape(-1), kc.view(np.uint8).reshape(-1))
    assert np.array_equal(cache_bytes(g.v_cache).reshape(-1), vc.view(np.uint8).reshape(-1))
    if window:
        bt = free_blocks_outside_window(w, window, sinks)
        ref = orc.decode(w.q, cfg.q_dtype, kc, vc, cfg.kv_dtype, bt, w.context_lens, w.scale, w.k_scale,
                         w.v_scale, window=window, sinks=sinks, threads=THREADS)
        out = torch.empty_like(g.out)
        pkv.paged_attention_decode_window(g.q, g.k_cache, g.v_cache, torch.from_numpy(bt).cuda(), g.context_lens,
                                          w.scale, out, w.max_context_len, window, sinks, partition_size=part,
                                          kv_dtype=g.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale,
                                          shared_blocks=bool(w.shared_blocks))
    else:
        out = g.decode(part)
    torch.cuda.synchronize()
    assert_close_to_oracle(out_to_f64(out), ref, cfg.kv_dtype, f"sweep case {i}")
