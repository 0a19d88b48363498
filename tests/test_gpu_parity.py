"""HIP path vs the oracle, through the C ABI (GPU only).

Bars: slot mapping and cache writes bit-exact; decode outputs within
4e-3 * max(1, |ref|) (2e-2 for fp8 KV) of the fp64 oracle, element by element.
"""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import (GpuStep, assert_close_to_oracle, cache_bytes, out_to_f64, to_device,
                         torch_dtype)
from helpers import oracle_step
from pins import SMALL
from workloads import CONFIGS, LLAMA8B, LONGCTX, R70B_FP8, TINY, make_workload

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _oracle_all(orc, w):
    return oracle_step(orc, w, threads=THREADS)


# ---------------------------------------------------------------- write --------
@pytest.mark.parametrize("name", sorted(SMALL))
def test_slots_and_write_bit_exact(orc, name):
    w = make_workload(SMALL[name])
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    torch.cuda.synchronize()
    kc, vc, ns, _ = _oracle_all(orc, w)
    if w.hist_seq.size:
        hs = orc.slot_mapping(w.hist_seq, w.hist_pos, w.block_tables, w.cfg.block_size)
        assert np.array_equal(g.hist_slots.cpu().numpy(), hs)
    assert np.array_equal(g.new_slots.cpu().numpy(), ns)
    assert np.array_equal(cache_bytes(g.k_cache).reshape(-1), kc.view(np.uint8).reshape(-1))
    assert np.array_equal(cache_bytes(g.v_cache).reshape(-1), vc.view(np.uint8).reshape(-1))


def test_write_fp8_every_bf16_input(orc):
    """All 65536 bf16 bit patterns (NaN, inf, subnormals, ties) quantised by the GPU
    write and by the oracle: identical fp8 bytes."""
    H, D, B = 2, 128, 16
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, H, D)
    for scale in (1.0, 0.0123, 3.5):
        nb = 256 // B
        kc = torch.full((nb, H, B, D), 0x7F, dtype=torch.uint8, device="cuda")
        vc = kc.clone()
        slots = torch.arange(256, dtype=torch.int64, device="cuda")
        k = to_device(codes, "bf16")
        v = to_device(codes[::-1].copy(), "bf16")
        pkv.paged_kv_write(slots, k, v, kc, vc, "fp8", scale, scale)
        kco = np.full((nb, H, B, D), 0x7F, np.uint8)
        vco = kco.copy()
        orc.kv_write(np.arange(256, dtype=np.int64), codes, codes[::-1].copy(), "bf16", kco, vco,
                     "fp8", scale, scale)
        assert np.array_equal(kc.cpu().numpy(), kco), scale
        assert np.array_equal(vc.cpu().numpy(), vco), scale


def test_write_fp8_f32_inputs(orc):
    """fp32 sources: random values over the whole e4m3 range, exact code values,
    midpoints (ties) and out-of-range values."""
    H, D, B = 1, 64, 16
    rng = np.random.default_rng(11)
    grid = orc.fp8_to_f64(np.arange(256, dtype=np.uint8))
    grid = np.unique(grid[np.isfinite(grid)])
    mids = (grid[1:] + grid[:-1]) / 2
    vals = np.concatenate([grid, mids, rng.uniform(-500, 500, 3000), rng.normal(0, 1, 3000),
                           [np.inf, -np.inf, np.nan, 1e30, -1e-30, 0.0, -0.0]]).astype(np.float32)
    n = (vals.size + D - 1) // D
    vals = np.resize(vals, n * D).reshape(n, H, D)
    nb = (n + B - 1) // B
    kc = torch.zeros((nb, H, B, D), dtype=torch.uint8, device="cuda")
    vc = kc.clone()
    slots = torch.arange(n, dtype=torch.int64, device="cuda")
    pkv.paged_kv_write(slots, to_device(vals, "f32"), to_device(vals, "f32"), kc, vc, "fp8", 1.0, 0.5)
    kco = np.zeros((nb, H, B, D), np.uint8)
    vco = kco.copy()
    orc.kv_write(np.arange(n, dtype=np.int64), vals, vals, "f32", kco, vco, "fp8", 1.0, 0.5)
    assert np.array_equal(kc.cpu().numpy(), kco)
    assert np.array_equal(vc.cpu().numpy(), vco)


@pytest.mark.parametrize("kind", ["negative", "past-the-cache"])
def test_slots_without_a_cache_row_skip(orc, kind):
    """Negative slots, and slots at or past num_blocks * B, write nothing."""
    w = make_workload(SMALL["llama8b"])
    g = GpuStep(w)
    c = w.cfg
    before = cache_bytes(g.k_cache).copy()
    before_v = cache_bytes(g.v_cache).copy()
    end = w.num_blocks * c.block_size
    vals = [-1, -2, -(1 << 40)] if kind == "negative" else [end, end + 1, end + c.block_size, 1 << 40]
    slots = torch.tensor([vals[i % len(vals)] for i in range(c.num_seqs)], dtype=torch.int64, device="cuda")
    pkv.paged_kv_write(slots, g.new_k, g.new_v, g.k_cache, g.v_cache)
    torch.cuda.synchronize()
    assert np.array_equal(cache_bytes(g.k_cache), before)
    assert np.array_equal(cache_bytes(g.v_cache), before_v)


@pytest.mark.parametrize("name", sorted(SMALL))
def test_write_positions_matches_slots_then_write(orc, name):
    """Slot resolution inside the write kernel: the caches come out bit-identical to the
    oracle's slot mapping followed by its write, and the returned slots are the oracle's.
    Tokens with no cache row (bad sequence ID or position) then write nothing."""
    w = make_workload(SMALL[name])
    g = GpuStep(w)
    c = w.cfg
    g.fill_history()
    slots = torch.full((c.num_seqs,), 7, dtype=torch.int64, device="cuda")
    pkv.paged_kv_write_positions(g.new_seq, g.new_pos, g.block_tables, g.new_k, g.new_v, g.k_cache, g.v_cache,
                                 g.kv_dtype, w.k_scale, w.v_scale, slot_mapping=slots)
    torch.cuda.synchronize()
    kc, vc, ns, _ = oracle_step(orc, w, pairs=np.zeros((0, 2), np.int32))
    assert np.array_equal(slots.cpu().numpy(), ns)
    assert np.array_equal(cache_bytes(g.k_cache).reshape(-1), kc.view(np.uint8).reshape(-1))
    assert np.array_equal(cache_bytes(g.v_cache).reshape(-1), vc.view(np.uint8).reshape(-1))
    # no cache row: a negative sequence ID or position, a position past the table's row
    nb = w.block_tables.shape[1]
    bad_seq = torch.tensor([(-1, 0, 0)[i % 3] for i in range(c.num_seqs)], dtype=torch.int32, device="cuda")
    bad_pos = torch.tensor([(5, -3, nb * c.block_size)[i % 3] for i in range(c.num_seqs)], dtype=torch.int32,
                           device="cuda")
    before_k, before_v = cache_bytes(g.k_cache).copy(), cache_bytes(g.v_cache).copy()
    pkv.paged_kv_write_positions(bad_seq, bad_pos, g.block_tables, g.new_k, g.new_v, g.k_cache, g.v_cache,
                                 g.kv_dtype, w.k_scale, w.v_scale, slot_mapping=slots)
    pkv.paged_kv_write_positions(bad_seq, bad_pos, g.block_tables, g.new_k, g.new_v, g.k_cache, g.v_cache,
                                 g.kv_dtype, w.k_scale, w.v_scale)  # no slot output
    torch.cuda.synchronize()
    assert np.all(slots.cpu().numpy() == -1)
    assert np.array_equal(cache_bytes(g.k_cache), before_k)
    assert np.array_equal(cache_bytes(g.v_cache), before_v)


def test_slot_mapping_without_a_table_entry(orc):
    """A negative position or sequence ID, or a position whose block index is past the
    table's row, maps to -1; the other tokens map as the oracle does."""
    w = make_workload(SMALL["llama8b"])
    c = w.cfg
    nb = w.block_tables.shape[1]
    seq = np.array([0, 1, 2, -1, 1, 0, 2, 1], np.int32)
    pos = np.array([0, 17, 5, 3, -4, nb * c.block_size, nb * c.block_size - 1, 1 << 30], np.int32)
    bad = (seq < 0) | (pos < 0) | (pos // c.block_size >= nb)
    got = pkv.paged_kv_slot_mapping(torch.from_numpy(seq).cuda(), torch.from_numpy(pos).cuda(),
                                    torch.from_numpy(w.block_tables).cuda(), c.block_size)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.all(got[bad] == -1)
    ref = orc.slot_mapping(seq[~bad], pos[~bad], w.block_tables, c.block_size)
    assert np.array_equal(got[~bad], ref)


# --------------------------------------------------------------- decode --------
@pytest.mark.parametrize("mode", [None, -1, "two-blocks"], ids=["default", "single", "split"])
@pytest.mark.parametrize("name", sorted(SMALL))
def test_decode_small(orc, name, mode):
    w = make_workload(SMALL[name])
    part = 2 * w.cfg.block_size if mode == "two-blocks" else mode
    g = GpuStep(w)
    out = out_to_f64(g.run(part))
    _, _, _, ref = _oracle_all(orc, w)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, f"{name}/{mode}")


FULL_MODES = [(c, None) for c in CONFIGS] + [(LONGCTX, 0), (LLAMA8B, 512)]


@pytest.mark.parametrize("cfg,part", FULL_MODES,
                         ids=[f"{c.name}-{'default' if p is None else p}" for c, p in FULL_MODES])
def test_full_size(orc, cfg, part):
    """The workload at its full size, in the launch configuration the benchmark times
    (and the other schedule for two of them): the whole cache after the write is
    compared byte by byte, and every decode output against the oracle."""
    print(f"full-size case {cfg.name} seed {cfg.seed} partition {part}", flush=True)
    w = make_workload(cfg)
    g = GpuStep(w)
    out = out_to_f64(g.run(part))
    kc, vc, ns, _ = oracle_step(orc, w, pairs=np.zeros((0, 2), np.int32))
    assert np.array_equal(g.new_slots.cpu().numpy(), ns)
    assert np.array_equal(cache_bytes(g.k_cache).reshape(-1), kc.view(np.uint8).reshape(-1))
    assert np.array_equal(cache_bytes(g.v_cache).reshape(-1), vc.view(np.uint8).reshape(-1))
    del g
    c = w.cfg
    ref = orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype, w.block_tables, w.context_lens,
                     w.scale, w.k_scale, w.v_scale, threads=THREADS)
    assert_close_to_oracle(out, ref, c.kv_dtype, cfg.name)


# ----------------------------------------------------------- invariances --------
@pytest.mark.parametrize("name", ["prefix", "r70b", "llama8b"])
def test_physical_permutation_bit_identical(name):
    """Moving every block to another physical ID (tables rewritten) gives bit-identical output."""
    w = make_workload(SMALL[name])
    g = GpuStep(w)
    out1 = g.run().clone()
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.num_blocks)).cuda()
    inv = torch.argsort(perm)
    g.k_cache = g.k_cache[inv].contiguous()  # new block perm[b] holds old block b
    g.v_cache = g.v_cache[inv].contiguous()
    g.block_tables = perm[g.block_tables.long()].to(torch.int32).contiguous()
    out2 = g.decode()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_split_matches_single():
    cfg = LLAMA8B.replace(num_seqs=6, ctx_params=(300, 1700), out_dtype="f32")
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    single = g.decode(-1).clone()
    for part in (16, 64, 512):
        split = g.decode(part).clone()
        torch.cuda.synchronize()
        assert (split - single).abs().max().item() <= 1e-5, part


@pytest.mark.parametrize("name", ["prefix", "r70b", "llama8b"])
def test_cache_policy_flag_bit_identical(name):
    """The shared-blocks flag only changes the load cache policy: outputs are bit-identical
    with and without it, in every schedule."""
    w = make_workload(SMALL[name])
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    for part in (0, -1, 2 * w.cfg.block_size):
        a = g.decode(part, shared_blocks=False).clone()
        b = g.decode(part, shared_blocks=True).clone()
        torch.cuda.synchronize()
        assert torch.equal(a, b), (name, part)


def test_workspace_reuse_keeps_header_zero():
    """One workspace serves balanced, fixed and balanced-again calls of different shapes:
    results match a fresh workspace each time and the counter header is zero after every
    call (the balanced kernel's arrival counters return to zero)."""
    hdr = pkv.WORKSPACE_HEADER_BYTES
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    for n, lo, hi, part in ((6, 300, 1700, 0), (40, 16, 4000, 0), (5, 100, 900, 64), (17, 1, 2500, 0),
                            (3, 9000, 12000, 0)):
        cfg = LLAMA8B.replace(num_seqs=n, ctx_params=(lo, hi), out_dtype="f32")
        g = GpuStep(make_workload(cfg))
        g.fill_history()
        g.write_new()
        for rep in range(3):
            got = g.decode(part, workspace=ws).clone()
            torch.cuda.synchronize()
            assert int(ws[:hdr].count_nonzero().item()) == 0, (n, part, rep)
            ref = g.decode(part).clone()  # fresh zeroed workspace from the binding
            torch.cuda.synchronize()
            assert torch.equal(got, ref), (n, part, rep)


# ------------------------------------------------------------- edge cases --------
EDGE = {
    "ctx-edges-b16": LLAMA8B.replace(num_seqs=9, ctx_kind="fixed",
                                     ctx_params=(1, 15, 16, 17, 31, 32, 33, 512, 513)),
    "ctx-edges-b32": LLAMA8B.replace(num_seqs=8, block_size=32, ctx_kind="fixed",
                                     ctx_params=(1, 16, 31, 32, 33, 64, 65, 1025)),
    "ctx-zero": LLAMA8B.replace(num_seqs=3, ctx_kind="fixed", ctx_params=(0, 5, 0)),
    "mha": LLAMA8B.replace(num_seqs=3, num_q_heads=4, num_kv_heads=4, ctx_params=(20, 300)),
    "g3": LLAMA8B.replace(num_seqs=3, num_q_heads=6, num_kv_heads=2, ctx_params=(20, 300)),
    "g16": LLAMA8B.replace(num_seqs=3, num_q_heads=32, num_kv_heads=2, ctx_params=(20, 300)),
    "mqa-g8": LLAMA8B.replace(num_seqs=3, num_q_heads=8, num_kv_heads=1, ctx_params=(20, 300)),
    "d64-bf16": LLAMA8B.replace(num_seqs=3, head_dim=64, ctx_params=(20, 300)),
    "f16": LLAMA8B.replace(num_seqs=3, q_dtype="f16", kv_dtype="f16", src_dtype="f16",
                           out_dtype="f16", ctx_params=(20, 300)),
    "fp8-f16q": R70B_FP8.replace(num_seqs=3, q_dtype="f16", src_dtype="f16", out_dtype="f16",
                                 ctx_params=(100, 0.8, 16, 600)),
    "fp8-d64-b32": R70B_FP8.replace(num_seqs=3, head_dim=64, block_size=32, num_q_heads=16,
                                    ctx_params=(100, 0.8, 16, 600)),
    "fp32-d128": TINY.replace(head_dim=128, pool_blocks=0),
    "fp8-out-f32": R70B_FP8.replace(num_seqs=3, out_dtype="f32", ctx_params=(100, 0.8, 16, 600)),
    "mix-zeros": LLAMA8B.replace(num_seqs=10, ctx_kind="fixed",
                                 ctx_params=(0, 1, 300, 0, 17, 1000, 16, 2, 4097, 33)),
    "many-seqs-short": LLAMA8B.replace(num_seqs=600, num_q_heads=8, num_kv_heads=2,
                                       ctx_params=(1, 40)),
    # 1100 sequences x 8 KV heads: many short contexts, every schedule
    "many-pairs-fixed": LLAMA8B.replace(num_seqs=1100, num_q_heads=8, num_kv_heads=8,
                                        ctx_params=(1, 90)),
}


@pytest.mark.parametrize("mode", [None, "two-blocks"], ids=["default", "split"])
@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(orc, name, mode):
    w = make_workload(EDGE[name])
    part = 2 * w.cfg.block_size if mode else None
    out = out_to_f64(GpuStep(w).run(part))
    _, _, _, ref = _oracle_all(orc, w)
    assert_close_to_oracle(out, ref, w.cfg.kv_dtype, name)
    if name == "ctx-zero":
        assert (out[0] == 0).all() and (out[2] == 0).all()


def test_empty_batch():
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((0, 1), dtype=torch.int32, device="cuda")
    cl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    pkv.paged_attention_decode(q, kc, kc, bt, cl, 0.1, out, 0)


def test_fp8_value_codes_exact(orc):
    """One cached token whose V holds every finite e4m3fn code: with one token the weight
    is exactly 1, so out (fp32) = code * v_scale exactly.  A NaN code gives NaN in its
    own output dim (the block-diagonal P.V product may spread a non-finite V element to
    the other dims of its group of 4; finite values are unaffected)."""
    H, D, B = 2, 128, 16
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[(codes & 0x7F) != 0x7F]  # 254 codes
    vcodes = np.concatenate([finite, finite[:2]]).reshape(H, D)
    for vc_row, nan_dim in ((vcodes, None), (np.where(np.arange(H * D).reshape(H, D) == 77, 0x7F, vcodes).astype(np.uint8), 77)):
        kc = np.full((2, H, B, D), 0x7F, np.uint8)
        vc = kc.copy()
        kc[1, :, 0, :] = 0x38  # K = 1.0
        vc[1, :, 0, :] = vc_row
        bt = np.array([[1]], np.int32)
        cl = np.array([1], np.int32)
        q = np.random.default_rng(1).standard_normal((1, 4, D)).astype(np.float32)
        qb = torch.from_numpy(q).to(torch.bfloat16)
        out = torch.empty((1, 4, D), dtype=torch.float32, device="cuda")
        pkv.paged_attention_decode(qb.cuda(), torch.from_numpy(kc).cuda(), torch.from_numpy(vc).cuda(),
                                   torch.from_numpy(bt).cuda(), torch.from_numpy(cl).cuda(), 0.1, out,
                                   1, kv_dtype="fp8", k_scale=0.5, v_scale=0.25)
        got = out.cpu().numpy().astype(np.float64)
        qbits = qb.view(torch.int16).numpy().view(np.uint16)
        ref = orc.decode(qbits, "bf16", kc, vc, "fp8", bt, cl, 0.1, 0.5, 0.25)
        if nan_dim is None:
            assert np.array_equal(got, ref)  # one fp32 rounding of an exact product
        else:
            assert np.isnan(got[0, :2, nan_dim]).all()  # query heads 0, 1 read KV head 0
            group = (np.arange(D) // 4) == nan_dim // 4
            assert np.array_equal(got[0, :2, ~group], ref[0, :2, ~group])
            assert np.array_equal(got[0, 2:], ref[0, 2:])
