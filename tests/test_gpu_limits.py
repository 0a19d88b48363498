"""Decode at the limits of its schedules, through the C ABI (GPU only), against the
oracle within the decode bar (4e-3 * max(1, |ref|)):

* 8 191 sequences, the most the balanced schedule takes (its per-sequence chunk prefix
  fills the largest LDS array it allocates);
* 8 192 sequences, one past it: the library's choice falls back to fixed partitions (one
  pass for contexts within a partition, partitions and the merge kernel beyond);
* one 262 144-token context: in the balanced schedule a single segment spans every
  workgroup, so the last workgroup to finish combines one partial from each of them; in
  512-token partitions the merge kernel combines 512 partials; in one pass a single
  workgroup per KV head streams it all;
* shared-prefix decode of 8 191 sequences, and a single 4 096-token prefill chunk.

The schedule each case runs is checked first, so a change of the planning rules cannot
silently move a case off the path it is meant to cover.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, out_to_f64
from helpers import oracle_step
from workloads import LLAMA8B, make_workload

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _check(orc, cfg, partition, schedule):
    w = make_workload(cfg)
    g = GpuStep(w)
    plan = pkv.paged_attention_schedule(pkv.cache_desc(g.k_cache), cfg.q_dtype, cfg.num_seqs, cfg.num_q_heads,
                                        w.max_context_len, partition)
    print(f"limits case {cfg.name}: N={cfg.num_seqs} max ctx={w.max_context_len} partition={partition} "
          f"plan={plan}", flush=True)
    assert plan["schedule"] == schedule, plan
    out = out_to_f64(g.run(partition))
    _, _, _, ref = oracle_step(orc, w, threads=THREADS)
    assert_close_to_oracle(out, ref, cfg.kv_dtype, cfg.name)
    return plan


def test_most_sequences_balanced(orc):
    cfg = LLAMA8B.replace(name="limits-8191-seqs", num_seqs=8191, num_q_heads=2, num_kv_heads=1,
                          ctx_params=(1, 48), seed=8191)
    _check(orc, cfg, 0, "balanced")


@pytest.mark.parametrize("hi,schedule", [(400, "single-pass"), (1100, "fixed-partitions")],
                         ids=["one-pass", "partitions"])
def test_one_sequence_past_balanced(orc, hi, schedule):
    cfg = LLAMA8B.replace(name=f"limits-8192-seqs-{hi}", num_seqs=8192, num_q_heads=2, num_kv_heads=1,
                          ctx_params=(1, hi), seed=8192 + hi)
    plan = _check(orc, cfg, 0, schedule)
    if schedule == "fixed-partitions":
        assert plan["partition"] == 512, plan


@pytest.mark.parametrize("partition,schedule", [(0, "balanced"), (512, "fixed-partitions"), (-1, "single-pass")],
                         ids=["balanced", "p512", "one-pass"])
def test_longest_context(orc, partition, schedule):
    cfg = LLAMA8B.replace(name="limits-256k-context", num_seqs=1, num_q_heads=4, num_kv_heads=1,
                          ctx_kind="fixed", ctx_params=(262144,), seed=262144)
    _check(orc, cfg, partition, schedule)


def test_shared_prefix_most_sequences(orc):
    """8 191 sequences on one shared prefix: the suffix pass's per-sequence LDS arrays at
    their largest beside its prefix-partial tiles."""
    from workloads import PREFIX
    cfg = PREFIX.replace(name="limits-prefix-8191-seqs", num_seqs=8191, num_q_heads=4, num_kv_heads=1,
                         ctx_params=(64, 0, 20), seed=18191)
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    starts = torch.from_numpy(np.asarray(w.prefix_group_starts(), np.int32)).cuda()
    pl = torch.full((cfg.num_seqs,), 64, dtype=torch.int32, device="cuda")
    print(f"limits case {cfg.name}: N={cfg.num_seqs} groups={list(w.prefix_group_starts())}", flush=True)
    pkv.paged_attention_decode_shared_prefix(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale,
                                             g.out, w.max_context_len, starts, pl, cfg.num_seqs, 64,
                                             kv_dtype=g.kv_dtype)
    torch.cuda.synchronize()
    _, _, _, ref = oracle_step(orc, w, threads=THREADS)
    assert_close_to_oracle(out_to_f64(g.out), ref, cfg.kv_dtype, cfg.name)


def test_prefill_whole_4096_token_prompt(orc):
    """One 4 096-token chunk, the whole prompt (32 row tiles of 128 rows per KV head)."""
    from gpu_helpers import to_device, torch_dtype
    from workloads import prefill_queries
    cfg = LLAMA8B.replace(name="limits-prefill-4096", num_seqs=1, num_q_heads=4, num_kv_heads=1,
                          ctx_kind="fixed", ctx_params=(4096,), seed=4096)
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    q, cu = prefill_queries(w, (4096,), 11)
    out = torch.empty((4096, cfg.num_q_heads, cfg.head_dim), dtype=torch_dtype(cfg.out_dtype), device="cuda")
    print(f"limits case {cfg.name}: one 4096-token chunk", flush=True)
    pkv.paged_attention_prefill(to_device(q, cfg.q_dtype), torch.from_numpy(cu).cuda(), 4096, g.k_cache, g.v_cache,
                                g.block_tables, g.context_lens, w.scale, out, w.max_context_len)
    torch.cuda.synchronize()
    got = out_to_f64(out)
    del g
    kc, vc, _, _ = oracle_step(orc, w, pairs=np.zeros((0, 2), np.int32))
    ref = orc.prefill(q, cfg.q_dtype, cu, kc, vc, cfg.kv_dtype, w.block_tables, w.context_lens, w.scale,
                      w.k_scale, w.v_scale, threads=THREADS)
    assert_close_to_oracle(got, ref, cfg.kv_dtype, cfg.name)
