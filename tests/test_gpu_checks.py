"""The library's input checks on the GPU against the oracle's rules (oracle/checks.py),
through the C ABI.  Results are integers, so they must agree exactly: the number of
violations, the lowest code and its lowest index.

* seeded random sweeps: index arrays drawn around their valid ranges (out-of-range
  IDs, negative and overlong lengths, duplicates, broken groupings), sized from empty to
  several 256-entry tiles with ragged ends;
* the generated workloads at their full sizes break no rule;
* debug mode (PAGEDKV_DEBUG=1): a call whose inputs break a rule raises
  PreconditionError and launches nothing; valid calls run as without it.

Only the checks read the broken inputs: no attention or write kernel is given an index
that would take it outside its buffers.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from gpu_helpers import GpuStep, out_to_f64, to_device
from oracle import checks as C
from workloads import CONFIGS, EXTRA_CONFIGS, LLAMA8B, PREFIX, make_workload, prefill_queries

pytestmark = pytest.mark.gpu
N_CASES = 40


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load_library()


def _cache(num_blocks, block_size, heads=2, dim=64):
    """A small cache tensor: the checks read only its shape (block count, block size)."""
    return torch.empty((num_blocks, heads, block_size, dim), dtype=torch.bfloat16, device="cuda")


def _dev(a, dtype=np.int32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).cuda()


def _sizes(rng):
    return int(rng.choice([0, 1, 5, 63, 64, 255, 256, 257, 600, 1100]))


@pytest.mark.parametrize("i", range(N_CASES))
def test_slot_and_position_checks_sweep(i):
    rng = np.random.default_rng(500 + i)
    B = int(rng.choice([16, 32]))
    nb = int(rng.integers(1, 40))
    rows = nb * B
    n = _sizes(rng)
    kc = _cache(nb, B)
    slots = rng.integers(-3, rows + 3, n).astype(np.int64)
    print(f"check sweep {i}: slots n={n} rows={rows}", flush=True)
    got = tuple(pkv.paged_kv_check_slots(_dev(slots, np.int64), kc))
    assert got == C.check_slots(slots, nb, B), (i, got)
    ns = int(rng.integers(0, 20))
    mb = int(rng.integers(1, 9))
    bt = rng.integers(-2, nb + 2, (ns, mb)).astype(np.int32)
    seq = rng.integers(-2, ns + 2, n).astype(np.int32)
    pos = rng.integers(-2, mb * B + 5, n).astype(np.int32)
    print(f"check sweep {i}: positions n={n} seqs={ns} max_blocks={mb}", flush=True)
    got = tuple(pkv.paged_kv_check_positions(_dev(seq), _dev(pos), _dev(bt), kc))
    assert got == C.check_positions(seq, pos, ns, bt, nb, B), (i, got)


def _tables_and_contexts(rng, ns, B, nb, max_ctx, bad=0.1):
    mb = -(-max_ctx // B)
    ctx = rng.integers(0, max_ctx + 1, ns).astype(np.int32)
    flip = rng.random(ns) < bad
    ctx[flip] = rng.choice([-3, -1, max_ctx + 1, max_ctx + 7], int(flip.sum()))
    bt = rng.integers(0, nb, (ns, mb)).astype(np.int32)
    bad_ids = rng.random((ns, mb)) < bad / 4
    bt[bad_ids] = rng.choice([-1, -7, nb, nb + 3], int(bad_ids.sum()))
    return bt, ctx


@pytest.mark.parametrize("i", range(N_CASES))
def test_decode_and_prefill_checks_sweep(i):
    rng = np.random.default_rng(700 + i)
    B = int(rng.choice([16, 32]))
    nb = int(rng.integers(4, 200))
    ns = int(rng.choice([0, 1, 3, 4, 5, 17, 64, 300]))
    max_ctx = int(rng.integers(1, 1500))
    bt, ctx = _tables_and_contexts(rng, ns, B, nb, max_ctx, bad=float(rng.choice([0.0, 0.05, 0.3])))
    window = int(rng.choice([0, 0, 1, 17, 300]))
    sinks = int(rng.choice([0, 1, 4, 40])) if window else 0
    kc = _cache(nb, B)
    print(f"check sweep {i}: decode seqs={ns} B={B} blocks={nb} max_ctx={max_ctx} window={window} sinks={sinks}",
          flush=True)
    got = tuple(pkv.paged_attention_check_decode(_dev(bt), _dev(ctx), max_ctx, kc, window=window, sinks=sinks))
    assert got == C.check_decode(bt, ctx, max_ctx, nb, B, window, sinks), (i, got)
    max_q = int(rng.integers(0, max_ctx + 1))
    n = rng.integers(0, max_q + 2, ns)
    n[rng.random(ns) < 0.1] = -2
    cu = np.concatenate([[int(rng.choice([0, 0, 0, 1]))], np.cumsum(n)]).astype(np.int32)
    print(f"check sweep {i}: prefill max_q_len={max_q}", flush=True)
    got = tuple(pkv.paged_attention_check_prefill(_dev(cu), max_q, _dev(bt), _dev(ctx), max_ctx, kc))
    assert got == C.check_prefill(cu, max_q, bt, ctx, max_ctx, nb, B), (i, got)


@pytest.mark.parametrize("i", range(N_CASES))
def test_shared_prefix_checks_sweep(i):
    rng = np.random.default_rng(900 + i)
    B = int(rng.choice([16, 32]))
    nb = int(rng.integers(8, 300))
    ns = int(rng.choice([1, 2, 7, 40, 300]))
    max_ctx = B * int(rng.integers(2, 40))
    bt, ctx = _tables_and_contexts(rng, ns, B, nb, max_ctx, bad=float(rng.choice([0.0, 0.0, 0.05])))
    ng = int(rng.integers(1, min(ns, 6) + 1))
    cuts = np.sort(rng.choice(np.arange(1, ns), ng - 1, replace=False)) if ng > 1 else np.zeros(0, int)
    gs = np.concatenate([[0], cuts, [ns]]).astype(np.int32)
    max_prefix = B * int(rng.integers(0, max_ctx // B + 1))
    pl = np.zeros(ns, np.int32)
    for j in range(ng):  # a valid grouping: equal prefixes, shared entries copied from the first
        f, e = gs[j], gs[j + 1]
        p = B * int(rng.integers(0, max_prefix // B + 1))
        p = min(p, int(ctx[f:e].clip(0).min()) // B * B)
        pl[f:e] = p
        bt[f + 1:e, :p // B] = bt[f, :p // B]
    max_group = int(np.diff(gs).max())
    r = rng.random()
    if r < 0.2:  # break the grouping
        k = int(rng.integers(0, ng + 1))
        gs[k] += int(rng.choice([-2, -1, 1, 3]))
    elif r < 0.5:  # break prefix lengths
        for s in rng.choice(ns, min(ns, 3), replace=False):
            pl[s] += int(rng.choice([-B, -1, 1, B, 2 * B]))
    elif r < 0.8:  # break shared entries
        for s in rng.choice(ns, min(ns, 3), replace=False):
            if pl[s] >= B:
                bt[s, int(rng.integers(0, pl[s] // B))] = int(rng.integers(0, nb))
    if rng.random() < 0.2:
        max_group = max(1, max_group - 1)
    kc = _cache(nb, B)
    print(f"check sweep {i}: shared prefix seqs={ns} groups={list(gs)} max_prefix={max_prefix} "
          f"max_group={max_group}", flush=True)
    got = tuple(pkv.paged_attention_check_shared_prefix(_dev(bt), _dev(ctx), max_ctx, _dev(gs), _dev(pl),
                                                        max_group, max_prefix, kc))
    assert got == C.check_shared_prefix(bt, ctx, max_ctx, nb, B, gs, max_group, pl, max_prefix), (i, got)


@pytest.mark.parametrize("i", range(N_CASES))
def test_block_id_checks_sweep(i):
    rng = np.random.default_rng(1100 + i)
    nb = int(rng.integers(1, 3000))
    n = _sizes(rng)
    dst = rng.integers(-2, nb + 2, n).astype(np.int32)
    src = rng.integers(-2, nb + 2, n).astype(np.int32) if rng.random() < 0.6 else None
    kc = _cache(nb, 16)
    print(f"check sweep {i}: block IDs n={n} blocks={nb} sources={src is not None}", flush=True)
    got = tuple(pkv.paged_kv_check_block_ids(_dev(src) if src is not None else None, _dev(dst), kc))
    assert got == C.check_block_ids(src, dst, nb), (i, got)


@pytest.mark.parametrize("cfg", CONFIGS + EXTRA_CONFIGS, ids=lambda c: c.name)
def test_workloads_pass_every_check(cfg):
    w = make_workload(cfg)
    g = GpuStep(w)
    kd = g.kv_dtype
    none = pkv.CheckResult(0, 0, -1)
    print(f"check workload {cfg.name}", flush=True)
    assert pkv.paged_attention_check_decode(g.block_tables, g.context_lens, w.max_context_len, g.k_cache,
                                            window=cfg.window, sinks=cfg.sinks, kv_dtype=kd) == none
    assert pkv.paged_kv_check_positions(g.new_seq, g.new_pos, g.block_tables, g.k_cache, kv_dtype=kd) == none
    slots = pkv.paged_kv_slot_mapping(g.new_seq, g.new_pos, g.block_tables, cfg.block_size)
    assert pkv.paged_kv_check_slots(slots, g.k_cache, kv_dtype=kd) == none
    if cfg.ctx_kind == "prefix":
        gs = torch.from_numpy(np.asarray(w.prefix_group_starts(), np.int32)).cuda()
        p = int(cfg.ctx_params[0])
        pl = torch.full((cfg.num_seqs,), p, dtype=torch.int32, device="cuda")
        mg = int(np.diff(np.asarray(w.prefix_group_starts())).max())
        assert pkv.paged_attention_check_shared_prefix(g.block_tables, g.context_lens, w.max_context_len, gs, pl,
                                                       mg, p, g.k_cache, kv_dtype=kd) == none


def test_debug_mode_raises_before_launching(monkeypatch):
    monkeypatch.setenv("PAGEDKV_DEBUG", "1")
    cfg = LLAMA8B.replace(num_seqs=6, num_q_heads=8, num_kv_heads=2, ctx_params=(40, 300), seed=77)
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    torch.cuda.synchronize()
    k0 = g.k_cache.clone()
    # two tokens writing one slot
    slots = pkv.paged_kv_slot_mapping(g.new_seq, g.new_pos, g.block_tables, cfg.block_size)
    slots[3] = slots[1]
    with pytest.raises(pkv.PreconditionError) as e:
        pkv.paged_kv_write(slots, g.new_k, g.new_v, g.k_cache, g.v_cache)
    assert e.value.result == (1, 1, 3)
    # a sequence ID past the table; the table is a view of a padded one, so even a missed
    # check would read a valid row
    seq = g.new_seq.clone()
    seq[2] = cfg.num_seqs
    padded = torch.cat([g.block_tables, g.block_tables[:1]])
    with pytest.raises(pkv.PreconditionError) as e:
        pkv.paged_kv_write_positions(seq, g.new_pos, padded[:cfg.num_seqs], g.new_k, g.new_v, g.k_cache, g.v_cache)
    assert e.value.result == (1, 2, 2)
    # a copy onto its own source; repeated swap-in IDs
    with pytest.raises(pkv.PreconditionError):
        pkv.paged_kv_copy_blocks(_dev([5]), _dev([5]), g.k_cache, g.v_cache)
    buf = torch.zeros((2,) + tuple(g.k_cache.shape[1:]), dtype=g.k_cache.dtype, device="cuda")
    with pytest.raises(pkv.PreconditionError):
        pkv.paged_kv_swap_in(_dev([7, 7]), buf, buf, g.k_cache, g.v_cache)
    torch.cuda.synchronize()
    assert torch.equal(g.k_cache.view(torch.int16), k0.view(torch.int16)), "a refused call wrote the cache"
    # valid calls run as without debug mode
    out_dbg = out_to_f64(g.decode(0, out=torch.empty_like(g.out)))
    monkeypatch.setenv("PAGEDKV_DEBUG", "0")
    out_plain = out_to_f64(g.decode(0, out=torch.empty_like(g.out)))
    assert np.array_equal(out_dbg, out_plain)


def test_debug_mode_shared_prefix_and_prefill(monkeypatch):
    monkeypatch.setenv("PAGEDKV_DEBUG", "1")
    cfg = PREFIX.replace(name="debug-prefix", num_seqs=12, num_q_heads=8, num_kv_heads=2, ctx_params=(128, 0, 60),
                         prefix_groups=2, seed=78)
    w = make_workload(cfg)
    g = GpuStep(w)
    g.fill_history()
    g.write_new()
    gs = _dev(w.prefix_group_starts())
    pl = torch.full((cfg.num_seqs,), 128, dtype=torch.int32, device="cuda")
    mg = int(np.diff(np.asarray(w.prefix_group_starts())).max())
    bt = g.block_tables.clone()
    s = int(w.prefix_group_starts()[0]) + 1
    bt[s, 1] = int(g.block_tables[s, 2])  # an in-range block, but not the shared one
    out = torch.full_like(g.out, float("nan"))
    with pytest.raises(pkv.PreconditionError) as e:
        pkv.paged_attention_decode_shared_prefix(g.q, g.k_cache, g.v_cache, bt, g.context_lens, w.scale, out,
                                                 w.max_context_len, gs, pl, mg, 128)
    assert e.value.result == (1, 7, s * bt.shape[1] + 1)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all(), "a refused call wrote its output"
    pkv.paged_attention_decode_shared_prefix(g.q, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale,
                                             out, w.max_context_len, gs, pl, mg, 128)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any()
    # prefill: more query rows than max_q_len (its grid would miss them)
    chunks = np.minimum(w.context_lens, 9)
    q, cu = prefill_queries(w, chunks, 3)
    qt = to_device(q, cfg.q_dtype)
    rows = torch.full((int(cu[-1]), cfg.num_q_heads, cfg.head_dim), float("nan"), dtype=torch.bfloat16,
                      device="cuda")
    with pytest.raises(pkv.PreconditionError) as e:
        pkv.paged_attention_prefill(qt, _dev(cu), 8, g.k_cache, g.v_cache, g.block_tables, g.context_lens, w.scale,
                                    rows, w.max_context_len)
    assert e.value.result.code == 8
    torch.cuda.synchronize()
    assert torch.isnan(rows.float()).all()


def test_duplicate_checks_at_prefill_scale():
    """The pairwise duplicate rules on 40 000 entries (a long prefill chunk's slots, a large
    copy-on-write batch): exact against the oracle, and quick enough for a debugging aid."""
    import time
    rng = np.random.default_rng(4242)
    nb, B, n = 4096, 16, 40000
    kc = _cache(nb, B)
    slots = rng.permutation(nb * B)[:n].astype(np.int64)
    slots[[123, 39000]] = slots[[7, 20000]]  # two duplicates, of earlier entries
    dev = _dev(slots, np.int64)
    pkv.paged_kv_check_slots(dev, kc)  # warm
    t = time.perf_counter()
    got = tuple(pkv.paged_kv_check_slots(dev, kc))
    ms = (time.perf_counter() - t) * 1e3
    print(f"slot check over {n} tokens: {ms:.1f} ms", flush=True)
    assert got == C.check_slots(slots, nb, B) == (2, C.DUPLICATE_SLOT, 123)
    assert ms < 1000
    dst = rng.permutation(nb)[: nb // 2].astype(np.int32)
    src = rng.permutation(nb)[: nb // 2].astype(np.int32)
    src = np.where(np.isin(src, dst), -1, src).astype(np.int32)  # sources never destinations ...
    src[5] = dst[900]  # ... but one
    dst = np.tile(dst, 20)[:n]
    src = np.tile(src, 20)[:n]
    got = tuple(pkv.paged_kv_check_block_ids(_dev(src), _dev(dst), kc))
    assert got == C.check_block_ids(src, dst, nb), got
