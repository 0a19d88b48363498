"""A decode step captured into a HIP graph (torch.cuda.graph) and replayed, through the C
ABI (GPU only).  Every library call is ordered on its stream, reads no device memory from
the host and allocates nothing when the caller brings the workspace, so a captured step
must give the eager results on every replay.

Each case captures the write of the new tokens (slot resolution inside the write kernel)
and one attention call -- decode under each schedule, fp8 decode, shared-prefix decode,
chunked prefill, or the no-alloc decode -- into one graph, then replays it three times.
Before each replay new query / key / value values (negated, halved or rolled over
sequences, so they stay within the fp8 scales) are copied into the graph's input tensors
and the caches are snapshotted.  After the replay the caches are set back to the snapshot
and the same calls run eagerly with their own output and workspace; then:
  * the replay's output is bit-identical to the eager output (same kernels and schedule,
    and the merges are deterministic);
  * the caches after the replay are byte-identical to those after the eager write;
  * the workspace's counter header is zero again after the replay;
  * the first replay, on the workload's own inputs, is within the decode bar of the oracle.
Between replays only eager work and synchronisations run; nothing in the graphs clears
memory with a memset.  A last case captures an input check (through the C ABI, which
neither waits nor allocates) and plants different out-of-range block IDs before each
replay: every replay reports the tables as they are then, exactly as the oracle's rules.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, out_to_f64, to_device, torch_dtype
from helpers import oracle_step
from workloads import LLAMA8B, PREFIX, R70B_FP8, make_workload, prefill_queries

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _variant(x: torch.Tensor, r: int) -> torch.Tensor:
    """Replay r's values of an input: the original, negated, or halved and rolled over
    the first dimension.  Exact in every dtype and never larger in magnitude."""
    if r == 0:
        return x.clone()
    if r == 1:
        return -x
    return torch.roll(x * 0.5, 1, 0)


def _bytes(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.uint8).clone()


class Step:
    """The static tensors of one captured step and the calls it makes."""

    def __init__(self, cfg, attend, ws_bytes=lambda desc, w: 0, out_shape=None):
        """ws_bytes(desc, workload): the workspace the attention call needs."""
        self.w = make_workload(cfg)
        self.g = GpuStep(self.w)
        self.g.fill_history()
        self.attend = attend  # attend(step, out, workspace)
        self.inputs = [self.g.q, self.g.new_k, self.g.new_v]
        self.originals = [x.clone() for x in self.inputs]
        shape = out_shape or tuple(self.g.out.shape)
        c = self.w.cfg
        self.out = torch.empty(shape, dtype=torch_dtype(c.out_dtype), device="cuda")
        self.out_eager = torch.empty_like(self.out)
        self.desc = pkv.cache_desc(self.g.k_cache, self.g.kv_dtype, self.w.k_scale, self.w.v_scale)
        n = max(ws_bytes(self.desc, self.w), 256)
        self.ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
        self.ws_eager = torch.zeros(n, dtype=torch.uint8, device="cuda")

    def write(self):
        g, w = self.g, self.w
        pkv.paged_kv_write_positions(g.new_seq, g.new_pos, g.block_tables, g.new_k, g.new_v, g.k_cache,
                                     g.v_cache, g.kv_dtype, w.k_scale, w.v_scale)

    def calls(self, out, ws):
        self.write()
        self.attend(self, out, ws)


def _replay_and_compare(step: Step, what: str, warm: bool = True):
    g = step.g
    if warm:  # per-device set-up (occupancy queries) outside capture
        step.calls(step.out_eager, step.ws_eager)
        torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.calls(step.out, step.ws)
    torch.cuda.synchronize()
    first = None
    for r in range(REPLAYS):
        for x, x0 in zip(step.inputs, step.originals):
            x.copy_(_variant(x0, r))
        k0, v0 = g.k_cache.clone(), g.v_cache.clone()
        torch.cuda.synchronize()
        print(f"graph case {what}: replay {r}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        out_g, kg, vg = _bytes(step.out), _bytes(g.k_cache), _bytes(g.v_cache)
        header = step.ws[:pkv.WORKSPACE_HEADER_BYTES]
        assert not bool(header.any()), f"{what} replay {r}: workspace header not zero"
        if r == 0:
            first = out_to_f64(step.out)
        g.k_cache.copy_(k0)
        g.v_cache.copy_(v0)
        step.calls(step.out_eager, step.ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out_g, _bytes(step.out_eager)), f"{what} replay {r}: output differs from eager"
        assert torch.equal(kg, _bytes(g.k_cache)), f"{what} replay {r}: K cache differs from eager"
        assert torch.equal(vg, _bytes(g.v_cache)), f"{what} replay {r}: V cache differs from eager"
        if r:
            assert not torch.equal(out_g, prev), f"{what} replay {r}: the new inputs were not read"
        prev = out_g
    del graph
    return first


def _decode_attend(part):
    def attend(step, out, ws):
        g, w = step.g, step.w
        pkv.paged_attention_decode(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale, out,
                                   w.max_context_len, partition_size=part, workspace=ws, kv_dtype=g.kv_dtype,
                                   k_scale=w.k_scale, v_scale=w.v_scale, shared_blocks=bool(w.shared_blocks))
    return attend


def _decode_ws(part):
    def ws(desc, w):
        c = w.cfg
        return pkv.paged_attention_workspace_size(desc, c.q_dtype, c.num_seqs, c.num_q_heads, w.max_context_len,
                                                  part)
    return ws


DECODE_CASES = {
    "balanced-bf16": (LLAMA8B.replace(num_seqs=16, num_q_heads=8, num_kv_heads=2, ctx_params=(100, 2500),
                                      seed=31), 0, "balanced"),
    "partitions-256-bf16": (LLAMA8B.replace(num_seqs=16, num_q_heads=8, num_kv_heads=2,
                                            ctx_params=(100, 2500), seed=32), 256, "fixed-partitions"),
    "one-pass-bf16": (LLAMA8B.replace(num_seqs=16, num_q_heads=8, num_kv_heads=2, ctx_params=(100, 2500),
                                      seed=33), -1, "single-pass"),
    "balanced-fp8": (R70B_FP8.replace(num_seqs=12, num_q_heads=16, num_kv_heads=2,
                                      ctx_params=(400, 0.8, 16, 2000), seed=34), 0, "balanced"),
}


@pytest.mark.parametrize("name", sorted(DECODE_CASES))
def test_graph_decode_step(orc, name):
    cfg, part, schedule = DECODE_CASES[name]
    step = Step(cfg, _decode_attend(part), _decode_ws(part))
    plan = pkv.paged_attention_schedule(step.desc, cfg.q_dtype, cfg.num_seqs, cfg.num_q_heads,
                                        step.w.max_context_len, part)
    assert plan["schedule"] == schedule, plan
    first = _replay_and_compare(step, name)
    _, _, _, ref = oracle_step(orc, step.w, threads=THREADS)
    assert_close_to_oracle(first, ref, cfg.kv_dtype, f"graph case {name}")


def test_graph_shared_prefix_step(orc):
    cfg = PREFIX.replace(name="graph-prefix", num_seqs=24, num_q_heads=8, num_kv_heads=2,
                         ctx_params=(256, 0, 100), prefix_groups=2, seed=35)
    w0 = make_workload(cfg)
    starts_np = np.asarray(w0.prefix_group_starts(), np.int32)
    starts = torch.from_numpy(starts_np).cuda()
    pl = torch.full((cfg.num_seqs,), 256, dtype=torch.int32, device="cuda")
    max_group = int(np.diff(starts_np).max())

    def attend(step, out, ws):
        g, w = step.g, step.w
        pkv.paged_attention_decode_shared_prefix(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale,
                                                 out, w.max_context_len, starts, pl, max_group, 256, workspace=ws,
                                                 kv_dtype=g.kv_dtype)

    def ws(desc, w):
        return pkv.paged_attention_shared_prefix_workspace_size(desc, cfg.q_dtype, cfg.num_seqs, cfg.num_q_heads,
                                                                w.max_context_len, len(starts_np) - 1, max_group,
                                                                256)

    step = Step(cfg, attend, ws)
    assert step.ws.numel() > 256
    first = _replay_and_compare(step, "shared-prefix")
    _, _, _, ref = oracle_step(orc, step.w, threads=THREADS)
    assert_close_to_oracle(first, ref, cfg.kv_dtype, "graph case shared-prefix")


def test_graph_prefill_step(orc):
    cfg = LLAMA8B.replace(name="graph-prefill", num_seqs=3, num_q_heads=8, num_kv_heads=2, ctx_kind="fixed",
                          ctx_params=(300, 41, 170), seed=36)
    chunks = (120, 41, 1)
    w0 = make_workload(cfg)
    q_np, cu_np = prefill_queries(w0, chunks, 37)
    cu = torch.from_numpy(cu_np).cuda()
    rows = int(cu_np[-1])

    def attend(step, out, ws):
        g, w = step.g, step.w
        pkv.paged_attention_prefill(step.q_rows, cu, max(chunks), g.k_cache, g.v_cache, g.block_tables,
                                    g.context_lens, w.scale, out, w.max_context_len, kv_dtype=g.kv_dtype)

    step = Step(cfg, attend, out_shape=(rows, cfg.num_q_heads, cfg.head_dim))
    step.q_rows = to_device(q_np, cfg.q_dtype)
    step.inputs = [step.q_rows, step.g.new_k, step.g.new_v]
    step.originals = [x.clone() for x in step.inputs]
    first = _replay_and_compare(step, "prefill")
    kc, vc, _, _ = oracle_step(orc, step.w, pairs=np.zeros((0, 2), np.int32))
    ref = orc.prefill(q_np, cfg.q_dtype, cu_np, kc, vc, cfg.kv_dtype, step.w.block_tables, step.w.context_lens,
                      step.w.scale, step.w.k_scale, step.w.v_scale, threads=THREADS)
    assert_close_to_oracle(first, ref, cfg.kv_dtype, "graph case prefill")


def test_graph_noalloc_step(orc):
    """The no-alloc decode, captured with no eager no-alloc call before it (in a process
    where nothing has used it yet this is its first use on the GPU, which records the
    scratch header's one-time clear into the graph).  Its output is compared with the
    eager workspace decode's, bit for bit."""
    cfg = LLAMA8B.replace(num_seqs=16, num_q_heads=8, num_kv_heads=2, ctx_params=(100, 2500), seed=38)
    decode = _decode_attend(0)

    def attend(step, out, workspace):
        g, w = step.g, step.w
        if workspace is step.ws:  # the captured call
            pkv.paged_attention_decode_noalloc(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale,
                                               out, w.max_context_len, partition_size=0)
        else:
            decode(step, out, workspace)

    step = Step(cfg, attend, _decode_ws(0))
    step.calls(step.out_eager, step.ws_eager)  # the workspace decode's set-up, outside capture
    torch.cuda.synchronize()
    first = _replay_and_compare(step, "no-alloc", warm=False)
    _, _, _, ref = oracle_step(orc, step.w, threads=THREADS)
    assert_close_to_oracle(first, ref, cfg.kv_dtype, "graph case no-alloc")


def test_graph_input_check_replays():
    """An input check captured through the C ABI (no memset, no synchronisation, it clears
    its own result): each replay reports the tables as they are at that replay."""
    import ctypes
    from oracle import checks as C
    from paged_kv_cache_27_amd._checks import _lib, RESULT_BYTES
    w = make_workload(LLAMA8B.replace(num_seqs=16, num_q_heads=8, num_kv_heads=2, ctx_params=(100, 2500),
                                      seed=39))
    g = GpuStep(w)
    desc = pkv.cache_desc(g.k_cache)
    bt = g.block_tables.clone()
    res = torch.zeros(RESULT_BYTES, dtype=torch.uint8, device="cuda")
    lib = _lib()
    pkv.paged_attention_check_decode(bt, g.context_lens, w.max_context_len, g.k_cache)  # set-up outside capture
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st = lib.paged_attention_check_decode(w.cfg.num_seqs,
                                              ctypes.byref(desc), bt.data_ptr(), bt.shape[1],
                                              g.context_lens.data_ptr(), w.max_context_len, 0, 0, res.data_ptr(),
                                              torch.cuda.current_stream().cuda_stream)
    assert st == 0
    rng = np.random.default_rng(40)
    for r in range(4):
        table = w.block_tables.copy()
        for _ in range(r):  # r planted out-of-range IDs among the entries the decode reads
            s = int(rng.integers(w.cfg.num_seqs))
            table[s, int(rng.integers(-(-int(w.context_lens[s]) // w.cfg.block_size)))] = w.num_blocks + r
        bt.copy_(torch.from_numpy(table))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        raw = res.cpu().numpy()
        got = (int(raw[16:24].view(np.int64)[0]), int(raw[0:4].view(np.int32)[0]), int(raw[8:16].view(np.int64)[0]))
        want = C.check_decode(table, w.context_lens, w.max_context_len, w.num_blocks, w.cfg.block_size)
        print(f"graph case input check: replay {r}: {got}", flush=True)
        assert got == want, (r, got, want)
        eager = pkv.paged_attention_check_decode(bt, g.context_lens, w.max_context_len, g.k_cache)
        assert tuple(eager) == want
    del graph
