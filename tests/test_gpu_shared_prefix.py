"""Shared-prefix (cascade) decode vs the oracle, through the C ABI (GPU only).

The entry point must compute exactly what plain decode computes; the bar is the same
(4e-3 * max(1, |ref|) against the fp64 oracle, element by element; 2e-2 over fp8
caches).  The groupings
passed to it vary independently of how the cache actually shares blocks, as long as
the declared sharing is real: the true grouping, finer groups, a shorter declared
prefix, singleton groups without a prefix, and prefixes that cover whole contexts.
"""
import dataclasses
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, out_to_f64
from helpers import oracle_step
from workloads import LLAMA8B, PREFIX, make_workload

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _run(g, starts, prefix_lens, out=None, workspace=None, scale=None):
    w = g.w
    scale = w.scale if scale is None else scale
    starts = np.asarray(starts, np.int32)
    prefix_lens = np.asarray(prefix_lens, np.int32)
    gmax = int(np.diff(starts).max())
    pmax = int(prefix_lens.max())
    out = g.out if out is None else out
    pkv.paged_attention_decode_shared_prefix(
        g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, scale, out, w.max_context_len,
        torch.from_numpy(starts).cuda(), torch.from_numpy(prefix_lens).cuda(), gmax, pmax,
        workspace=workspace, kv_dtype=g.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    torch.cuda.synchronize()
    return out


def _true_grouping(w):
    starts = w.prefix_group_starts()
    prefix = int(w.cfg.ctx_params[0])
    return starts, np.full(w.cfg.num_seqs, prefix, np.int32)


def _prepared(cfg):
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    return w, g


CASES = {
    "one-group": PREFIX.replace(num_seqs=6, ctx_params=(128, 0, 70)),
    "three-groups": PREFIX.replace(num_seqs=11, prefix_groups=3, ctx_params=(96, 0, 90)),
    "b16-f32out": PREFIX.replace(num_seqs=9, block_size=16, prefix_groups=2, ctx_params=(80, 0, 60),
                                 out_dtype="f32"),
    "f16-d64": PREFIX.replace(num_seqs=5, head_dim=64, q_dtype="f16", kv_dtype="f16", src_dtype="f16",
                              out_dtype="f16", ctx_params=(64, 0, 50)),
    "mqa-g8": PREFIX.replace(num_seqs=7, num_q_heads=8, num_kv_heads=1, ctx_params=(64, 0, 33)),
    "mha-g1": PREFIX.replace(num_seqs=5, num_q_heads=4, num_kv_heads=4, ctx_params=(96, 0, 40)),
    "g3": PREFIX.replace(num_seqs=6, num_q_heads=12, num_kv_heads=4, ctx_params=(64, 0, 40)),
    "many-rows": PREFIX.replace(num_seqs=80, prefix_groups=2, ctx_params=(192, 0, 45)),
    "fp8-bf16q": PREFIX.replace(num_seqs=11, prefix_groups=3, kv_dtype="fp8", ctx_params=(96, 0, 90)),
    "fp8-f16q-d64-g8": PREFIX.replace(num_seqs=7, head_dim=64, num_q_heads=8, num_kv_heads=1, q_dtype="f16",
                                      kv_dtype="fp8", out_dtype="f16", ctx_params=(64, 0, 33)),
    # G x slices = 16 (4 slices of a 64-token prefix; 8 of a 128-token one at G = 2): the
    # suffix pass takes the prefix partials into LDS at a segment's first piece.  (The
    # cases above with G x slices > 16 or G > 4 fold them from memory.)
    "fp8-lds-fold": PREFIX.replace(num_seqs=9, prefix_groups=2, kv_dtype="fp8", ctx_params=(64, 0, 70)),
    "g2-lds-fold": PREFIX.replace(num_seqs=5, num_q_heads=16, num_kv_heads=8, block_size=16,
                                  ctx_params=(128, 0, 40)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_true_grouping_matches_oracle(orc, name):
    w, g = _prepared(CASES[name])
    starts, pl = _true_grouping(w)
    print(f"shared-prefix case {name}: groups {list(starts)} prefix {pl[0]}", flush=True)
    out = out_to_f64(_run(g, starts, pl))
    _, _, _, ref = oracle_step(orc, w, threads=THREADS)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, name)


@pytest.mark.parametrize("scale", [-0.0883883, 0.0])
def test_scale_values(orc, scale):
    """A negative softmax scale and a zero one: the prefix partials and the suffix pass
    must use the same log2-domain maxima for the merge to hold."""
    w, g = _prepared(CASES["three-groups"])
    starts, pl = _true_grouping(w)
    print(f"shared-prefix scale {scale}", flush=True)
    out = out_to_f64(_run(g, starts, pl, scale=scale))
    _, _, _, ref = oracle_step(orc, dataclasses.replace(w, scale=scale), threads=THREADS)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, f"scale {scale}")


def test_declared_groupings(orc):
    """Valid groupings other than the true one all give the oracle's result: finer groups,
    a shorter declared prefix, no prefix at all, and a mix."""
    w, g = _prepared(CASES["three-groups"])
    _, _, _, ref = oracle_step(orc, w, threads=THREADS)
    starts, pl = _true_grouping(w)
    assert list(starts) == [0, 3, 7, 11]
    n, B = w.cfg.num_seqs, w.cfg.block_size
    variants = {
        "finer": ([0, 1, 3, 5, 7, 9, 11], pl),  # refines the true groups [0, 3, 7, 11]
        "shorter-prefix": (starts, np.full(n, B, np.int32)),
        "no-prefix": (list(range(n + 1)), np.zeros(n, np.int32)),
        "mixed": ([0, 2, 3, 4, 7, 11], np.array([96, 96, 0, 0, 64, 64, 64, 96, 96, 96, 96], np.int32)),
    }
    for name, (st, p) in variants.items():
        out = out_to_f64(_run(g, st, p))
        assert_close_to_oracle(out, ref, w.cfg.kv_dtype, name)


def test_prefix_covering_whole_contexts(orc):
    """Singleton groups whose declared prefix is the whole context (a block multiple):
    the suffix pass has nothing to stream and the output is the prefix alone."""
    cfg = LLAMA8B.replace(num_seqs=6, ctx_kind="fixed", ctx_params=(16, 48, 64, 33, 160, 17))
    w, g = _prepared(cfg)
    _, _, _, ref = oracle_step(orc, w, threads=THREADS)
    ctx = w.context_lens
    pl = (ctx // 16 * 16).astype(np.int32)  # 16, 48, 64, 32, 160, 16
    out = out_to_f64(_run(g, list(range(7)), pl))
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, "whole-context prefixes")


def test_agrees_with_plain_decode_and_is_deterministic():
    w, g = _prepared(CASES["three-groups"].replace(out_dtype="f32"))
    starts, pl = _true_grouping(w)
    a = _run(g, starts, pl).clone()
    b = _run(g, starts, pl).clone()
    assert torch.equal(a, b)
    plain = g.decode(0).clone()
    torch.cuda.synchronize()
    assert (a - plain).abs().max().item() <= 1e-4


def test_workspace_reuse_keeps_header_zero():
    w, g = _prepared(CASES["many-rows"].replace(out_dtype="f32"))
    starts, pl = _true_grouping(w)
    ws = torch.zeros(128 << 20, dtype=torch.uint8, device="cuda")
    ref = _run(g, starts, pl).clone()
    for _ in range(3):
        got = _run(g, starts, pl, workspace=ws).clone()
        assert int(ws[:pkv.WORKSPACE_HEADER_BYTES].count_nonzero().item()) == 0
        assert torch.equal(got, ref)
        g.decode(0, workspace=ws)  # the plain balanced decode shares the workspace
        torch.cuda.synchronize()
        assert int(ws[:pkv.WORKSPACE_HEADER_BYTES].count_nonzero().item()) == 0


def test_full_size_prefix_workload(orc):
    """The 256-sequence prefix-sharing workload at full size through the shared-prefix
    entry point (the benchmark's launch), every output against the oracle."""
    w, g = _prepared(PREFIX)
    starts, pl = _true_grouping(w)
    out = out_to_f64(_run(g, starts, pl))
    del g
    c = w.cfg
    kc, vc, _, _ = oracle_step(orc, w, pairs=np.zeros((0, 2), np.int32))
    ref = orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype, w.block_tables, w.context_lens, w.scale,
                     w.k_scale, w.v_scale, threads=THREADS)
    assert_close_to_oracle(out, ref, c.kv_dtype, c.name)
