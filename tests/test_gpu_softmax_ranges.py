"""Decode on score ranges that drive the online softmax's rescaling (GPU only).

The decoders keep a reference maximum per head that moves only when a chunk's maximum
exceeds it by more than 2^8 in weight; random N(0,1) data rarely moves it after the first
chunk.  Here the K rows are built so that the scores climb steeply (the reference moves on
every chunk, then many tokens share the top), fall steeply (it never moves and later
weights underflow), or the softmax scale is large; every output is compared with the fp64
oracle element by element (4e-3 * max(1, |ref|)), in the default and split schedules.
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, out_to_f64
from helpers import oracle_step
from workloads import LLAMA8B, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def _shaped(cfg, ramp):
    """The workload with each token's K row (per KV head) along its group's mean query
    direction, scaled so that the scores follow ramp(position, context) in log2 units of
    the softmax weight (plus small noise)."""
    w = make_workload(cfg)
    c = w.cfg
    G, D = c.num_q_heads // c.num_kv_heads, c.head_dim
    q = _bits_f32(w.q).reshape(c.num_seqs, c.num_kv_heads, G, D).astype(np.float64)
    u = q.mean(axis=2)
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    proj = np.einsum("sghd,sgd->sgh", q, u).mean(axis=2)  # typical q . u per (seq, KV head)
    c_l2 = abs(w.scale) / np.log(2.0)
    rng = np.random.default_rng(5)

    def rows(seq, pos):
        target = np.array([ramp(p, w.context_lens[s]) for s, p in zip(seq, pos)])  # log2 units
        a = target[:, None] / (c_l2 * proj[seq])  # [T][H_kv]
        k = a[:, :, None] * u[seq] + 0.05 * rng.standard_normal((len(seq), c.num_kv_heads, D))
        return _bf16_bits(k)

    w.hist_k = rows(w.hist_seq, w.hist_pos)
    w.new_k = rows(w.new_seq, w.new_pos)
    return w


CFG = LLAMA8B.replace(num_seqs=4, ctx_kind="fixed", ctx_params=(700, 333, 90, 17), out_dtype="f32")
CASES = {
    # +9 log2 units per 16 tokens over the first 64 tokens, flat after: the reference max
    # moves on each of those chunks, then hundreds of tokens share the top weight
    "rising": (CFG, lambda p, n: 9.0 / 16.0 * min(p, 64)),
    # the same over a long context split across many workgroups
    "rising-long": (LLAMA8B.replace(num_seqs=2, ctx_kind="fixed", ctx_params=(3000, 1500), out_dtype="f32"),
                    lambda p, n: 9.0 / 16.0 * min(p, 64)),
    # -2 log2 units per token: the maximum is in the first chunk, later weights underflow
    "falling": (CFG, lambda p, n: -2.0 * p),
}


@pytest.mark.parametrize("mode", [None, "two-blocks"], ids=["default", "split"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_score_ramps(orc, name, mode):
    cfg, ramp = CASES[name]
    print(f"softmax ramp {name} mode {mode}", flush=True)
    w = _shaped(cfg, ramp)
    part = 2 * w.cfg.block_size if mode else None
    out = out_to_f64(GpuStep(w).run(part))
    _, _, _, ref = oracle_step(orc, w)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, name)


@pytest.mark.parametrize("mode", [None, "two-blocks"], ids=["default", "split"])
def test_negative_scale_on_a_ramp(orc, mode):
    """A negative scale flips the ramp: the first tokens weigh most."""
    print(f"softmax negative scale mode {mode}", flush=True)
    w = _shaped(CFG, CASES["rising"][1])
    w = dataclasses.replace(w, scale=-w.scale)
    part = 2 * w.cfg.block_size if mode else None
    out = out_to_f64(GpuStep(w).run(part))
    _, _, _, ref = oracle_step(orc, w)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, "negative scale")


@pytest.mark.parametrize("mode", [None, "two-blocks"], ids=["default", "split"])
def test_large_scale(orc, mode):
    """Random data under a scale 64 times the usual one: weights spread over ~2^80."""
    print(f"softmax large scale mode {mode}", flush=True)
    w = make_workload(CFG)
    w = dataclasses.replace(w, scale=64.0 * w.scale)
    part = 2 * w.cfg.block_size if mode else None
    out = out_to_f64(GpuStep(w).run(part))
    _, _, _, ref = oracle_step(orc, w)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, "large scale")
