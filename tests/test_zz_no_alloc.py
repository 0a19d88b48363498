"""The no-alloc decode entry point (paged_attention_decode_noalloc), through the C ABI,
against paged_attention_decode with a caller-provided workspace.  Both run the same
schedule and kernels on the same inputs, so their outputs must be bit-identical.  Each
case makes calls in a row on the GPU's one scratch array -- a larger input, then a
smaller one, then the larger one again -- so stale counters or partials left by one call
would show in the next."""
import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep
from workloads import LLAMA8B, LONGCTX, R70B_FP8, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _ready(cfg):
    g = GpuStep(make_workload(cfg))
    g.fill_history()
    g.write_new()
    return g


def _noalloc(g, part):
    w = g.w
    out = torch.empty_like(g.out)
    pkv.paged_attention_decode_noalloc(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale, out,
                                       w.max_context_len, partition_size=part, kv_dtype=g.kv_dtype,
                                       k_scale=w.k_scale, v_scale=w.v_scale, shared_blocks=bool(w.shared_blocks))
    return out


SEQUENCES = {
    # balanced schedule: per-workgroup partials and arrival counters in the scratch
    "balanced-bf16": (0, [LLAMA8B.replace(num_seqs=24, ctx_params=(100, 3000)),
                          LLAMA8B.replace(num_seqs=5, ctx_params=(20, 600), seed=7)]),
    "balanced-fp8": (0, [R70B_FP8.replace(num_seqs=20, ctx_params=(500, 0.8, 16, 2000)),
                         R70B_FP8.replace(num_seqs=4, ctx_params=(60, 0.5, 16, 200), seed=8)]),
    # fixed partitions merged in the decode kernel: partials and per-(sequence, KV head)
    # counters in the scratch
    "fixed-512": (512, [LONGCTX.replace(num_seqs=2, ctx_params=(12000,)),
                        LONGCTX.replace(num_seqs=1, ctx_params=(3000,), seed=9)]),
    "fixed-64": (64, [LLAMA8B.replace(num_seqs=12, ctx_params=(300, 2000)),
                      LLAMA8B.replace(num_seqs=3, ctx_params=(65, 400), seed=10)]),
}


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_matches_decode_on_consecutive_calls(name):
    part, cfgs = SEQUENCES[name]
    steps = [_ready(c) for c in cfgs]
    for i, g in enumerate(steps + steps[:1]):  # larger, smaller, larger again
        print(f"no-alloc case {name} call {i}: {g.w.cfg.num_seqs} seqs, partition {part}", flush=True)
        got = _noalloc(g, part)
        ref = g.decode(part, out=torch.empty_like(g.out))  # fresh zero-headed workspace
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all(), (name, i)
        assert torch.equal(got, ref), (name, i)


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call whose schedule needs more than the scratch holds is refused with
    PKV_ERR_SCRATCH before anything is launched; the next call still works."""
    g = _ready(LLAMA8B.replace(num_seqs=4, ctx_params=(100, 400)))
    n, hq, d = 4000, 32, 128
    q = torch.zeros((n, hq, d), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((n, 256), dtype=torch.int32, device="cuda")
    cl = torch.ones(n, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    need = pkv.paged_attention_workspace_size(pkv.cache_desc(g.k_cache), "bf16", n, hq, 4096, 16)
    assert need > pkv.NOALLOC_SCRATCH_BYTES
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.paged_attention_decode_noalloc(q, g.k_cache, g.v_cache, bt, cl, 0.1, out, 4096, partition_size=16)
    assert e.value.status == -9
    got = _noalloc(g, 0)
    ref = g.decode(0, out=torch.empty_like(g.out))
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
