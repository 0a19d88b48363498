"""Whole-block moves (copy-on-write, swap) and the block lifecycle, through the C ABI
(GPU only).  Caches are compared byte for byte with the oracle's; decodes within the
decode bar."""
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, assert_close_to_oracle, cache_bytes, out_to_f64, to_device
from helpers import oracle_step
from workloads import LLAMA8B, R70B_FP8, TINY, make_workload

pytestmark = pytest.mark.gpu
THREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _ids(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _prepared(orc, cfg):
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    torch.cuda.synchronize()
    kc, vc, _, _ = oracle_step(orc, w)
    return w, g, kc, vc


def _assert_caches_equal(g, kc, vc, what):
    assert np.array_equal(cache_bytes(g.k_cache).reshape(-1), kc.view(np.uint8).reshape(-1)), what
    assert np.array_equal(cache_bytes(g.v_cache).reshape(-1), vc.view(np.uint8).reshape(-1)), what


def _live_blocks(w):
    live = set()
    for s, ctx in enumerate(w.context_lens):
        live |= set(w.block_tables[s, :(int(ctx) + w.cfg.block_size - 1) // w.cfg.block_size].tolist())
    return sorted(live)


def _pool_for(w):
    """A library pool holding exactly the workload's live blocks (count 1 each)."""
    pool = pkv.BlockPoolHandle(w.num_blocks)
    every = pool.alloc(w.num_blocks)
    pool.release([b for b in every.tolist() if b not in set(_live_blocks(w))])
    return pool


# Block geometries: 32 KiB (whole rounds of the move kernel's 8 x 256 16-byte pieces), 16
# KiB fp8 and 12 KiB fp32 (a partial round only), 40 KiB (a whole round, then a partial
# one) and 96 KiB (three whole rounds).
COPY_CASES = {
    "bf16": LLAMA8B.replace(num_seqs=3, ctx_params=(40, 300)),
    "fp8": R70B_FP8.replace(num_seqs=3, ctx_params=(200, 0.5, 16, 400)),
    "f32-12k": TINY.replace(num_kv_heads=3, num_q_heads=6, pool_blocks=0),
    "bf16-40k": LLAMA8B.replace(num_seqs=3, num_kv_heads=5, num_q_heads=20, block_size=32, ctx_params=(40, 300)),
    "bf16-96k": LLAMA8B.replace(num_seqs=3, num_kv_heads=12, num_q_heads=24, block_size=32, ctx_params=(40, 300)),
}


@pytest.mark.parametrize("name", sorted(COPY_CASES))
def test_copy_blocks_bit_exact(orc, name):
    cfg = COPY_CASES[name]
    w, g, kc, vc = _prepared(orc, cfg)
    rng = np.random.default_rng(5)
    live, free = _live_blocks(w), [b for b in range(w.num_blocks) if b not in set(_live_blocks(w))]
    n = min(len(live), len(free), 9)
    src = rng.choice(live, size=n, replace=True).astype(np.int32)
    dst = rng.choice(free, size=n, replace=False).astype(np.int32)
    src[1] = -1  # skipped pairs: a negative ID, IDs at or past num_blocks
    src[2] = w.num_blocks
    dst[3] = w.num_blocks + 7
    print(f"copy case {cfg.kv_dtype}: {n} pairs", flush=True)
    pkv.paged_kv_copy_blocks(_ids(src), _ids(dst), g.k_cache, g.v_cache, g.kv_dtype)
    torch.cuda.synchronize()
    orc.copy_blocks(np.where(src < w.num_blocks, src, -1), np.where(dst < w.num_blocks, dst, -1), kc, vc)
    _assert_caches_equal(g, kc, vc, "copy_blocks")


SWAP_CASES = [("bf16", "device"), ("bf16", "pinned-host"), ("fp8", "pinned-host"), ("bf16-40k", "pinned-host")]


@pytest.mark.parametrize("kv,where", SWAP_CASES, ids=[f"{k}-{w}" for k, w in SWAP_CASES])
def test_swap_round_trip(orc, kv, where):
    """Swap out to buffers in device memory or straight to pinned host memory (the kernel
    moves the blocks across the host link: "Estrategia 2: swap" keeps an evicted session
    in CPU RAM), byte-compared with the oracle's swap-out; then swap in from the same
    buffers to other blocks, caches compared byte for byte."""
    if kv == "fp8":
        cfg = R70B_FP8.replace(ctx_params=(100, 0.5, 16, 300), num_seqs=2, pool_factor=3.0)
    elif kv == "bf16-40k":  # a block of one whole and one partial round of the move kernel
        cfg = COPY_CASES[kv].replace(num_seqs=2, ctx_params=(64, 200), pool_factor=3.0)
    else:
        cfg = LLAMA8B.replace(num_seqs=2, ctx_params=(64, 200), pool_factor=3.0)
    w, g, kc, vc = _prepared(orc, cfg)
    live = _live_blocks(w)
    free = [b for b in range(w.num_blocks) if b not in set(live)]
    ids = np.array(live[:5] + [-1, w.num_blocks], np.int32)  # the last two rows skipped
    shape = (ids.size,) + tuple(g.k_cache.shape[1:])
    if where == "device":
        kb = torch.zeros(shape, dtype=g.k_cache.dtype, device="cuda")
        vb = torch.zeros_like(kb)
    else:
        kb = torch.zeros(shape, dtype=g.k_cache.dtype, pin_memory=True)
        vb = torch.zeros(shape, dtype=g.k_cache.dtype, pin_memory=True)
        assert kb.is_pinned() and vb.is_pinned()
    print(f"swap case {kv} {where}: {ids.size} rows", flush=True)
    pkv.paged_kv_swap_out(_ids(ids), g.k_cache, g.v_cache, kb, vb, g.kv_dtype)
    torch.cuda.synchronize()
    k_ref, v_ref = orc.swap_out(np.where(ids < w.num_blocks, ids, -1), kc, vc)
    assert np.array_equal(cache_bytes(kb)[:5], k_ref.view(np.uint8)[:5])
    assert np.array_equal(cache_bytes(vb)[:5], v_ref.view(np.uint8)[:5])
    assert not cache_bytes(kb)[5:].any() and not cache_bytes(vb)[5:].any()  # skipped rows untouched
    back = np.array(free[:5] + [w.num_blocks + 3, -1], np.int32)
    pkv.paged_kv_swap_in(_ids(back), kb, vb, g.k_cache, g.v_cache, g.kv_dtype)
    torch.cuda.synchronize()
    orc.swap_in(np.where(back < w.num_blocks, back, -1), k_ref, v_ref, kc, vc)
    _assert_caches_equal(g, kc, vc, "swap_in")


def test_swap_refuses_pageable_host_memory():
    """A pageable host buffer is refused before any launch (a kernel would fault on it)."""
    cfg = LLAMA8B.replace(num_seqs=1, ctx_kind="fixed", ctx_params=(40,), pool_blocks=8)
    w = make_workload(cfg)
    g = GpuStep(w)
    kb = torch.zeros((1,) + tuple(g.k_cache.shape[1:]), dtype=g.k_cache.dtype)  # pageable
    lib = pkv.load_library()
    import ctypes
    desc = pkv.cache_desc(g.k_cache)
    rc = lib.paged_kv_swap_out(_ids([0]).data_ptr(), 1, g.k_cache.data_ptr(), g.v_cache.data_ptr(),
                               ctypes.byref(desc), kb.data_ptr(), kb.data_ptr(), None)
    assert rc == -3
    with pytest.raises(ValueError):
        pkv.paged_kv_swap_out(_ids([0]), g.k_cache, g.v_cache, kb, kb)


def test_beam_fork_copy_on_write_then_decode(orc):
    """One 45-token prompt forked into 4 branches that share its 3 blocks.  Each branch
    writes its own next token: copy-on-write copies the last (partly filled) block for
    all branches but the last one to write, the full blocks stay shared.  Caches match
    the oracle byte for byte and the 4 branch decodes match the oracle."""
    cfg = LLAMA8B.replace(num_seqs=1, ctx_kind="fixed", ctx_params=(45,), pool_blocks=24)
    w, g, kc, vc = _prepared(orc, cfg)
    c, B = w.cfg, w.cfg.block_size
    pool = _pool_for(w)
    base = w.block_tables[0, :3].copy()
    for _ in range(3):
        pool.share(base)
    tables = np.tile(w.block_tables[0], (4, 1)).astype(np.int32)
    src, dst = [], []
    for b in range(4):
        new, copied = pool.cow(int(base[2]))
        if copied:
            src.append(int(base[2]))
            dst.append(new)
        tables[b, 2] = new
    assert len(src) == 3 and [pool.refcount(int(x)) for x in base[:2]] == [4, 4]
    pkv.paged_kv_copy_blocks(_ids(src), _ids(dst), g.k_cache, g.v_cache)
    orc.copy_blocks(np.array(src, np.int32), np.array(dst, np.int32), kc, vc)
    # every branch writes its own token 45 into its own last block
    rng = np.random.default_rng(9)
    knew = rng.standard_normal((4, c.num_kv_heads, c.head_dim)).astype(np.float32)
    vnew = rng.standard_normal((4, c.num_kv_heads, c.head_dim)).astype(np.float32)
    knew_b = torch.from_numpy(knew).to(torch.bfloat16)
    vnew_b = torch.from_numpy(vnew).to(torch.bfloat16)
    slots = tables[:, 2].astype(np.int64) * B + 45 % B
    pkv.paged_kv_write(torch.from_numpy(slots).cuda(), knew_b.cuda(), vnew_b.cuda(), g.k_cache, g.v_cache)
    kn = knew_b.view(torch.int16).numpy().view(np.uint16)
    vn = vnew_b.view(torch.int16).numpy().view(np.uint16)
    orc.kv_write(slots, kn, vn, "bf16", kc, vc, "bf16")
    torch.cuda.synchronize()
    _assert_caches_equal(g, kc, vc, "fork + copy-on-write + write")
    # the 4 branches decode with their own queries over 46 tokens
    q = torch.from_numpy(rng.standard_normal((4, c.num_q_heads, c.head_dim)).astype(np.float32)).to(torch.bfloat16)
    ctx = np.full(4, 46, np.int32)
    out = torch.empty((4, c.num_q_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")
    pkv.paged_attention_decode(q.cuda(), g.k_cache, g.v_cache, _ids(tables), _ids(ctx), w.scale, out, 46,
                               shared_blocks=True)
    torch.cuda.synchronize()
    qn = q.view(torch.int16).numpy().view(np.uint16)
    ref = orc.decode(qn, "bf16", kc, vc, "bf16", tables, ctx, w.scale)
    assert_close_to_oracle(out_to_f64(out), ref, "bf16", "beam branches")


def test_swap_out_reuse_swap_in_decodes_identically(orc):
    """Tiering: sequence 0 is swapped out to host memory, its blocks are released only
    after the transfer finished, reused (overwritten) by another session, and swapped
    back into fresh blocks: its decode is bit-identical to the decode before the swap,
    and matches the oracle."""
    cfg = LLAMA8B.replace(num_seqs=2, ctx_params=(100, 260), pool_factor=3.0)
    w, g, kc, vc = _prepared(orc, cfg)
    B = w.cfg.block_size
    pool = _pool_for(w)
    before = g.decode(0).clone()
    torch.cuda.synchronize()
    n0 = (int(w.context_lens[0]) + B - 1) // B
    ids0 = w.block_tables[0, :n0].copy()
    shape = (n0,) + tuple(g.k_cache.shape[1:])
    kb = torch.empty(shape, dtype=g.k_cache.dtype, device="cuda")
    vb = torch.empty_like(kb)
    pkv.paged_kv_swap_out(_ids(ids0), g.k_cache, g.v_cache, kb, vb)
    kh = torch.empty(shape, dtype=kb.dtype, pin_memory=True)
    vh = torch.empty(shape, dtype=kb.dtype, pin_memory=True)
    kh.copy_(kb, non_blocking=True)
    vh.copy_(vb, non_blocking=True)
    torch.cuda.synchronize()  # offload complete: only now may the GPU blocks go
    del kb, vb
    pool.release(ids0)
    other = pool.alloc(n0)  # another session takes (and overwrites) blocks
    junk = torch.full(shape, float("nan"), dtype=g.k_cache.dtype, device="cuda")
    pkv.paged_kv_swap_in(_ids(other), junk, junk, g.k_cache, g.v_cache)
    fresh = pool.alloc(n0)  # resume: new blocks, contents from host memory
    pkv.paged_kv_swap_in(_ids(fresh), kh.cuda(), vh.cuda(), g.k_cache, g.v_cache)
    bt = w.block_tables.copy()
    bt[0, :n0] = fresh
    g.block_tables = torch.from_numpy(bt).cuda()
    after = g.decode(0)
    torch.cuda.synchronize()
    assert torch.equal(after, before)
    c = w.cfg
    ref = orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype, w.block_tables, w.context_lens, w.scale)
    assert_close_to_oracle(out_to_f64(after), ref, c.kv_dtype, "after swap round trip")


def test_copy_blocks_full_size(orc):
    """1024 copy-on-write copies across the 8B-shaped layer's cache (64 KiB of K and V
    each), byte for byte."""
    w, g, kc, vc = _prepared(orc, LLAMA8B)
    live = _live_blocks(w)
    free = [b for b in range(w.num_blocks) if b not in set(live)]
    rng = np.random.default_rng(3)
    n = min(1024, len(free))
    src = rng.choice(live, size=n).astype(np.int32)
    dst = rng.choice(free, size=n, replace=False).astype(np.int32)
    print(f"full-size copy: {n} pairs", flush=True)
    pkv.paged_kv_copy_blocks(_ids(src), _ids(dst), g.k_cache, g.v_cache)
    torch.cuda.synchronize()
    orc.copy_blocks(src, dst, kc, vc)
    _assert_caches_equal(g, kc, vc, "full-size copy")
