"""Pins of the oracle to things other than itself.

Each pin raises AssertionError when the oracle disagrees with a value the pages
print, a closed form, a special case with a known answer, an invariant, or an
independent dense computation.  They are plain functions so that the mutation
test can run the same set against deliberately broken oracle builds.
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np
import torch

from helpers import (dense_causal, dense_reference, free_blocks_outside_window, oracle_step,
                     storage_to_f64)
from workloads import LLAMA8B, LONGCTX, PREFIX, R70B_FP8, TINY, make_workload, prefill_queries

GOLDEN = Path(__file__).resolve().parent / "golden"

# Small variants of the five workloads: same head geometry and dtypes, contexts
# short enough for fp64 loops, still spanning several blocks and a ragged tail.
SMALL = {
    "tiny": TINY,
    "llama8b": LLAMA8B.replace(num_seqs=3, ctx_params=(17, 70)),
    "r70b": R70B_FP8.replace(num_seqs=3, ctx_params=(48, 0.5, 16, 100)),
    "prefix": PREFIX.replace(num_seqs=4, ctx_params=(64, 0, 40)),
    "prefix-groups": PREFIX.replace(name="prefix-groups", num_seqs=7, prefix_groups=3,
                                    ctx_params=(64, 0, 40)),
    "longctx": LONGCTX.replace(num_seqs=2, ctx_params=(200,)),
    "mha-f16": TINY.replace(name="mha-f16", num_q_heads=4, num_kv_heads=4, q_dtype="f16",
                            kv_dtype="f16", src_dtype="f16", out_dtype="f16", pool_blocks=0,
                            ctx_kind="fixed", ctx_params=(1, 17, 48, 5)),
    "mqa": LLAMA8B.replace(name="mqa", num_seqs=2, num_q_heads=8, num_kv_heads=1,
                           ctx_params=(20, 60)),
}


def pin_kv_bytes_golden(orc):
    rows = json.loads((GOLDEN / "kv_bytes.json").read_text())["rows"]
    for r in rows:
        got = orc.kv_bytes(r["T"], r["L"], r["H_kv"], r["d_h"], r["b"])
        assert got == r["bytes"], (r, got)


def pin_block_addressing_golden(orc):
    g = json.loads((GOLDEN / "block_addressing.json").read_text())
    for ex in g["position_examples"]:
        B = ex["block_size"]
        table = np.arange(1000, 1000 + ex["logical_block"] + 1, dtype=np.int32)[None, :]
        slot = orc.slot_mapping([0], [ex["position"]], table, B)[0]
        assert slot // B == table[0, ex["logical_block"]], ex
        assert slot % B == ex["offset"], ex
    for ex in g["block_counts"]:
        B, n = ex["block_size"], ex["tokens"]
        nb = ex["blocks"] + 2
        table = (np.arange(nb, dtype=np.int32) * 7 + 3)[None, :]  # distinct physical IDs
        slots = orc.slot_mapping(np.zeros(n, np.int32), np.arange(n, dtype=np.int32), table, B)
        assert len(set((slots // B).tolist())) == ex["blocks"], ex
    t = g["table_example"]
    B = t["block_size"]
    table = np.asarray(t["block_table"], np.int32)[None, :]
    pos = np.arange(B * len(t["block_table"]), dtype=np.int32)
    slots = orc.slot_mapping(np.zeros(pos.size, np.int32), pos, table, B)
    assert (slots // B).reshape(-1, B)[:, 0].tolist() == t["expected_physical_by_logical_block"]
    assert ((slots % B).reshape(-1, B) == np.arange(B)).all()


def pin_dense_equivalence(orc, names=None):
    """Oracle over the paged cache == dense softmax(qK^T s)V over contiguous K/V."""
    for name in names or SMALL:
        w = make_workload(SMALL[name])
        _, _, _, out = oracle_step(orc, w)
        for s in range(w.cfg.num_seqs):
            ref = dense_reference(w, s)
            err = np.abs(out[s] - ref).max()
            assert err <= 1e-12, (name, s, err)


def pin_ctx1_returns_new_value(orc):
    """With one token in context, the softmax weight is 1: out == V of that token."""
    cfg = LLAMA8B.replace(num_seqs=3, ctx_kind="fixed", ctx_params=(1, 1, 1))
    w = make_workload(cfg)
    _, _, _, out = oracle_step(orc, w)
    v = storage_to_f64(w.new_v, "bf16")  # [N][H_kv][D]
    G = cfg.group
    for h in range(cfg.num_q_heads):
        assert np.array_equal(out[:, h, :], v[:, h // G, :]), h


def pin_equal_keys_mean_value(orc):
    """All keys equal -> uniform weights -> out == mean of V."""
    cfg = LLAMA8B.replace(num_seqs=2, ctx_params=(20, 45))
    w = make_workload(cfg)
    w.hist_k[:] = w.new_k[0:1]  # every token of every sequence gets the same key rows
    w.new_k[:] = w.new_k[0:1]
    # identical key per KV head across tokens (heads may differ)
    _, _, _, out = oracle_step(orc, w)
    G = cfg.group
    for s in range(cfg.num_seqs):
        _, v = w.logical_kv(s)
        vm = storage_to_f64(v, "bf16").mean(axis=0)
        for h in range(cfg.num_q_heads):
            assert np.abs(out[s, h] - vm[h // G]).max() <= 1e-12, (s, h)


def pin_zero_query_mean_value(orc):
    """q = 0 -> every score 0 -> out == mean of V."""
    cfg = TINY
    w = make_workload(cfg)
    w.q[:] = 0
    _, _, _, out = oracle_step(orc, w)
    G = cfg.group
    for s in range(cfg.num_seqs):
        _, v = w.logical_kv(s)
        vm = storage_to_f64(v, "f32").mean(axis=0)
        for h in range(cfg.num_q_heads):
            assert np.abs(out[s, h] - vm[h // G]).max() <= 1e-12, (s, h)


def pin_permutation_invariance(orc):
    """Moving blocks to other physical IDs (tables rewritten) leaves out bit-identical."""
    for name in ("tiny", "prefix", "r70b"):
        w = make_workload(SMALL[name])
        kc, vc, _, out = oracle_step(orc, w)
        rng = np.random.default_rng(7)
        perm = rng.permutation(w.num_blocks)  # old id -> new id
        kc2 = np.empty_like(kc)
        vc2 = np.empty_like(vc)
        kc2[perm] = kc
        vc2[perm] = vc
        bt2 = perm[w.block_tables].astype(np.int32)
        c = w.cfg
        out2 = orc.decode(w.q, c.q_dtype, kc2, vc2, c.kv_dtype, bt2, w.context_lens, w.scale,
                          w.k_scale, w.v_scale)
        assert np.array_equal(out, out2), name


def pin_gqa_head_mapping(orc):
    """Query head h reads KV head h // G: swapping two KV heads' data moves the outputs."""
    w = make_workload(SMALL["llama8b"])
    c = w.cfg
    kc, vc, _, out = oracle_step(orc, w)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, [0, 1]] = kc[:, [1, 0]]
    vc2[:, [0, 1]] = vc[:, [1, 0]]
    out2 = orc.decode(w.q, c.q_dtype, kc2, vc2, c.kv_dtype, w.block_tables, w.context_lens,
                      w.scale)
    G = c.group
    # heads of group 2.. unchanged; outputs of groups 0 and 1 change
    assert np.array_equal(out[:, 2 * G:], out2[:, 2 * G:])
    assert not np.array_equal(out[:, :G], out2[:, :G])


def pin_bytes_touched(orc):
    """The gather reads exactly each sequence's context once per query head:
    G * M_KV(sum ctx) with L = 1 (the closed form, 'Una formula util...')."""
    for name in ("tiny", "llama8b", "r70b", "prefix"):
        w = make_workload(SMALL[name])
        c = w.cfg
        kc, vc, _, _ = oracle_step(orc, w)
        _, nbytes = orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype, w.block_tables,
                               w.context_lens, w.scale, w.k_scale, w.v_scale, count_bytes=True)
        b = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}[c.kv_dtype]
        expect = c.group * orc.kv_bytes(int(w.context_lens.sum()), 1, c.num_kv_heads, c.head_dim, b)
        assert nbytes == expect, (name, nbytes, expect)
        assert nbytes == c.group * w.kv_bytes_algorithmic()


def pin_write_placement(orc):
    """After the write, exactly the written rows hold data; every other row is still poison;
    each written row equals the token's source (bit copy)."""
    w = make_workload(SMALL["llama8b"])
    c = w.cfg
    kc, vc, ns, _ = oracle_step(orc, w)
    poison = np.uint16(0x7FC0)
    live_rows = (kc != poison).any(axis=-1)  # [NB][H][B]
    n_tokens = w.hist_seq.size + c.num_seqs
    assert live_rows.sum() == n_tokens * c.num_kv_heads
    for s in range(c.num_seqs):
        blk, off = divmod(int(ns[s]), c.block_size)
        assert blk == w.block_tables[s, (w.context_lens[s] - 1) // c.block_size]
        assert off == (w.context_lens[s] - 1) % c.block_size
        assert np.array_equal(kc[blk, :, off, :], w.new_k[s])
        assert np.array_equal(vc[blk, :, off, :], w.new_v[s])


def pin_fp8_codec(orc):
    """e4m3fn decode of all 256 codes and RNE encode of in-range values vs torch's cast."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = orc.fp8_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    # Encode: every finite code value, every midpoint between neighbours (ties),
    # points a quarter of a step either side, and random values in range.
    vals = np.unique(ref[fin])
    mids = (vals[1:] + vals[:-1]) / 2
    steps = np.diff(vals)
    rng = np.random.default_rng(3)
    x = np.concatenate([vals, mids, mids + steps / 4, mids - steps / 4,
                        rng.uniform(-448, 448, 4000), rng.normal(0, 1, 4000),
                        rng.normal(0, 0.01, 2000)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.f32_to_fp8(x), want)


def pin_fp8_saturation(orc):
    """Beyond +-448 (including infinities) the encoder saturates; NaN stays NaN.
    (This is the chosen reading; the pages only say 'FP8'.)"""
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf], np.float32)
    assert orc.f32_to_fp8(x).tolist() == [0x7E] * 6 + [0xFE] * 2
    assert orc.f32_to_fp8(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F


def pin_half_codecs(orc):
    """bf16 and fp16 decoders vs torch over a spread of codes."""
    codes = np.arange(0, 65536, 97, dtype=np.uint32).astype(np.uint16)
    b_ref = torch.from_numpy(codes.astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    f_ref = torch.from_numpy(codes.astype(np.int16)).view(torch.float16).to(torch.float64).numpy()
    b = orc.bf16_to_f64(codes)
    f = orc.f16_to_f64(codes)
    for r, g in ((b_ref, b), (f_ref, f)):
        assert np.array_equal(np.isnan(r), np.isnan(g))
        assert np.array_equal(r[~np.isnan(r)], g[~np.isnan(g)])


# (window, sinks) cases: one token, within a block, a block, straddling blocks with 4
# sinks (the pages' count), sinks reaching past the window start, a window wider than
# any context.
WINDOW_CASES = [(1, 0), (5, 0), (16, 0), (17, 4), (33, 4), (20, 30), (4096, 4)]


def _decode_window(orc, w, kc, vc, window, sinks, tables=None):
    c = w.cfg
    return orc.decode(w.q, c.q_dtype, kc, vc, c.kv_dtype,
                      w.block_tables if tables is None else tables, w.context_lens, w.scale,
                      w.k_scale, w.v_scale, window=window, sinks=sinks)


def pin_window_dense(orc):
    """Windowed oracle == dense softmax over the explicitly selected rows (last `window`
    tokens plus the first `sinks`) of the contiguous K/V."""
    for name in ("llama8b", "r70b", "tiny", "mqa"):
        w = make_workload(SMALL[name])
        kc, vc, _, _ = oracle_step(orc, w)
        for W, S in WINDOW_CASES:
            out = _decode_window(orc, w, kc, vc, W, S)
            for s in range(w.cfg.num_seqs):
                err = np.abs(out[s] - dense_reference(w, s, W, S)).max()
                assert err <= 1e-12, (name, W, S, s, err)


def pin_window_one_is_last_value(orc):
    """A one-token window (no sinks) attends to the new token alone: out == its V."""
    w = make_workload(SMALL["llama8b"])
    kc, vc, _, _ = oracle_step(orc, w)
    out = _decode_window(orc, w, kc, vc, 1, 0)
    v = storage_to_f64(w.new_v, "bf16")
    G = w.cfg.group
    for h in range(w.cfg.num_q_heads):
        assert np.array_equal(out[:, h, :], v[:, h // G, :]), h


def pin_window_covering_is_full(orc):
    """A window as long as the context attends to everything: bit-identical to no window."""
    w = make_workload(SMALL["r70b"])
    kc, vc, _, full = oracle_step(orc, w)
    for W, S in ((int(w.context_lens.max()), 0), (int(w.context_lens.max()) + 5, 4)):
        assert np.array_equal(_decode_window(orc, w, kc, vc, W, S), full), (W, S)


def pin_window_freed_blocks_unread(orc):
    """Blocks holding no attended token may be freed (their table entries pointed at a
    NaN-filled block): the windowed output is unchanged, bit for bit."""
    w = make_workload(SMALL["llama8b"].replace(ctx_params=(60, 140)))
    kc, vc, _, _ = oracle_step(orc, w)
    for W, S in ((17, 4), (40, 0), (1, 16)):
        ref = _decode_window(orc, w, kc, vc, W, S)
        got = _decode_window(orc, w, kc, vc, W, S, free_blocks_outside_window(w, W, S))
        assert np.isfinite(got).all() and np.array_equal(got, ref), (W, S)


def _random_cache(rng, shape=(12, 2, 16, 64), dtype=np.uint16):
    return rng.integers(0, 2**16, size=shape, dtype=np.int64).astype(dtype)


def pin_copy_blocks(orc):
    """Copy-on-write copies == numpy's gather-then-assign of whole blocks, K and V each;
    pairs with a negative ID change nothing."""
    rng = np.random.default_rng(11)
    kc, vc = _random_cache(rng), _random_cache(rng)
    src = np.array([3, 7, 7, -1, 0], np.int32)
    dst = np.array([9, 1, 4, 5, 11], np.int32)
    k_ref, v_ref = kc.copy(), vc.copy()
    keep = (src >= 0) & (dst >= 0)
    k_ref[dst[keep]] = kc[src[keep]]
    v_ref[dst[keep]] = vc[src[keep]]
    orc.copy_blocks(src, dst, kc, vc)
    assert np.array_equal(kc, k_ref) and np.array_equal(vc, v_ref)


def pin_swap_round_trip(orc):
    """Swap out returns exactly the listed blocks; swapping them back into other blocks
    equals copying them there."""
    rng = np.random.default_rng(12)
    kc, vc = _random_cache(rng), _random_cache(rng)
    ids = np.array([2, 5, 8], np.int32)
    kb, vb = orc.swap_out(ids, kc, vc)
    assert np.array_equal(kb, kc[ids]) and np.array_equal(vb, vc[ids])
    k2, v2 = kc.copy(), vc.copy()
    orc.swap_in(np.array([10, 0, 3], np.int32), kb, vb, k2, v2)
    k3, v3 = kc.copy(), vc.copy()
    orc.copy_blocks(ids, np.array([10, 0, 3], np.int32), k3, v3)
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)


def _prefill(orc, w, kc, vc, q, cu, context_lens=None):
    c = w.cfg
    return orc.prefill(q, c.q_dtype, cu, kc, vc, c.kv_dtype, w.block_tables,
                       w.context_lens if context_lens is None else context_lens, w.scale, w.k_scale,
                       w.v_scale)


def pin_prefill_one_token_is_decode(orc):
    """A chunk of one token per sequence is a decode step: bit-identical outputs."""
    for name in ("llama8b", "r70b", "tiny"):
        w = make_workload(SMALL[name])
        kc, vc, _, dec = oracle_step(orc, w)
        cu = np.arange(w.cfg.num_seqs + 1, dtype=np.int32)
        assert np.array_equal(_prefill(orc, w, kc, vc, w.q, cu), dec), name


def pin_prefill_dense_causal(orc):
    """Each query token of a chunk == dense softmax over the contiguous K/V rows up to and
    including its own position (numpy, fp64), <= 1e-12."""
    for name, lens in (("llama8b", (9, 40, 1)), ("r70b", (16, 3, 33)), ("mqa", (20, 60))):
        w = make_workload(SMALL[name].replace(num_seqs=len(lens), ctx_kind="fixed",
                                              ctx_params=tuple(sorted(l + 30 for l in lens))))
        kc, vc, _, _ = oracle_step(orc, w)
        n = np.minimum(np.array(lens), w.context_lens)
        q, cu = prefill_queries(w, n)
        out = _prefill(orc, w, kc, vc, q, cu)
        c = w.cfg
        for s in range(c.num_seqs):
            for i in range(int(n[s])):
                pos = int(w.context_lens[s]) - int(n[s]) + i
                ref = dense_causal(w, s, q[cu[s] + i], pos)
                err = np.abs(out[cu[s] + i] - ref).max()
                assert err <= 1e-12, (name, s, i, err)


def pin_prefill_chunking_invariance(orc):
    """The outputs of a prompt's query tokens do not depend on how it is cut into chunks:
    one 40-token chunk == the same queries as a 25-token then a 15-token chunk (context
    grown between them), bit for bit."""
    w = make_workload(SMALL["llama8b"].replace(num_seqs=1, ctx_kind="fixed", ctx_params=(70,)))
    kc, vc, _, _ = oracle_step(orc, w)
    q, cu = prefill_queries(w, [40])
    whole = _prefill(orc, w, kc, vc, q, cu)
    first = _prefill(orc, w, kc, vc, q[:25], np.array([0, 25], np.int32), np.array([55], np.int32))
    second = _prefill(orc, w, kc, vc, q[25:], np.array([0, 15], np.int32))
    assert np.array_equal(np.concatenate([first, second]), whole)


ALL_PINS = [pin_kv_bytes_golden, pin_block_addressing_golden, pin_dense_equivalence,
            pin_ctx1_returns_new_value, pin_equal_keys_mean_value, pin_zero_query_mean_value,
            pin_permutation_invariance, pin_gqa_head_mapping, pin_bytes_touched,
            pin_write_placement, pin_fp8_codec, pin_fp8_saturation, pin_half_codecs,
            pin_window_dense, pin_window_one_is_last_value, pin_window_covering_is_full,
            pin_window_freed_blocks_unread, pin_copy_blocks, pin_swap_round_trip,
            pin_prefill_one_token_is_decode, pin_prefill_dense_causal, pin_prefill_chunking_invariance]
