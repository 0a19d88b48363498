"""Host-side block-pool fixture: the accounting and lifecycle invariants the pages list
("Capitulo 2", section "Evals deterministas para esta capa": Accounting, Lifecycle)."""
import numpy as np
import pytest

from workloads import CONFIGS, BlockPool, PREFIX, TINY, make_workload

SMALLISH = [c if c.num_seqs <= 8 and c.ctx_kind != "const" else
            c.replace(num_seqs=6, ctx_params=c.ctx_params if c.ctx_kind != "const" else (300,))
            for c in CONFIGS]


@pytest.mark.parametrize("cfg", SMALLISH, ids=lambda c: c.name)
def test_accounting(cfg):
    w = make_workload(cfg)
    B = cfg.block_size
    live = set()
    refs = np.zeros(w.num_blocks, np.int64)
    for s in range(cfg.num_seqs):
        n = (int(w.context_lens[s]) + B - 1) // B
        ids = w.block_tables[s, :n]
        live.update(ids.tolist())
        np.add.at(refs, ids, 1)
        # padding entries all point at the sentinel block
        assert (w.block_tables[s, n:] == w.sentinel_block).all()
    allocated = int((w.refcount > 0).sum())
    # allocated_blocks >= blocks referenced by live block tables
    assert allocated >= len(live)
    # free_blocks + allocated_blocks = pool_blocks
    assert allocated + len(w.free_blocks) == w.num_blocks
    assert set(w.free_blocks).isdisjoint(live | {w.sentinel_block})
    # reference counts equal the number of tables pointing at each live block
    for b in live:
        assert w.refcount[b] == refs[b]
    assert w.sentinel_block not in live


@pytest.mark.parametrize("cfg", SMALLISH, ids=lambda c: c.name)
def test_no_writable_aliasing(cfg):
    """The block each new token is written into is private (refcount 1): shared
    blocks are read-only, copy-on-write never has to trigger in a decode step."""
    w = make_workload(cfg)
    B = cfg.block_size
    targets = [int(w.block_tables[s, (w.context_lens[s] - 1) // B]) for s in range(cfg.num_seqs)]
    assert len(set(targets)) == len(targets)
    for b in targets:
        assert w.refcount[b] == 1
    # history rows: every (sequence, position) written exactly once
    keys = set(zip(w.hist_seq.tolist(), w.hist_pos.tolist()))
    assert len(keys) == w.hist_seq.size


def test_prefix_sharing_layout():
    w = make_workload(PREFIX.replace(num_seqs=5, ctx_params=(128, 0, 40)))
    shared_n = 128 // PREFIX.block_size
    for s in range(5):
        assert (w.block_tables[s, :shared_n] == w.block_tables[0, :shared_n]).all()
    assert (w.refcount[w.block_tables[0, :shared_n]] == 5).all()
    assert w.kv_bytes_unique() < w.kv_bytes_algorithmic()


def test_pool_lifecycle():
    rng = np.random.default_rng(0)
    pool = BlockPool(10, rng)
    a = [pool.allocate() for _ in range(4)]
    assert pool.num_free + pool.num_allocated == 10
    pool.share(a[0])
    pool.release(a[0])
    assert pool.refcount[a[0]] == 1  # still owned by the first holder
    for b in a:
        pool.release(b)
    assert pool.num_free == 10 and pool.num_allocated == 0
    with pytest.raises(AssertionError):
        pool.release(a[1])
    for _ in range(10):
        pool.allocate()
    with pytest.raises(RuntimeError):
        pool.allocate()


def test_tiny_shape():
    w = make_workload(TINY)
    assert w.num_blocks == 32
    assert w.context_lens.tolist() == [7, 16, 33, 100]
    # 1 + 1 + 3 + 7 live blocks
    assert sum((int(c) + 15) // 16 for c in w.context_lens) == 12


def test_prefix_groups_share_within_group_only():
    """Several prefix groups: each group's sequences share that group's prefix blocks
    (refcount = group size) and no block is shared across groups."""
    cfg = PREFIX.replace(num_seqs=7, prefix_groups=3, ctx_params=(64, 0, 40))
    w = make_workload(cfg)
    starts = w.prefix_group_starts()
    assert list(starts) == [0, 2, 4, 7]
    shared_n = 64 // cfg.block_size
    heads = []
    for j in range(3):
        a, b = starts[j], starts[j + 1]
        head = w.block_tables[a, :shared_n]
        for s in range(a, b):
            assert (w.block_tables[s, :shared_n] == head).all()
            assert w.prefix_owner(s) == a
        assert (w.refcount[head] == b - a).all()
        heads.append(set(head.tolist()))
    assert not (heads[0] & heads[1]) and not (heads[1] & heads[2]) and not (heads[0] & heads[2])
    # private blocks are private: every other live block has refcount 1
    live = set(w.block_tables[w.block_tables != w.sentinel_block].tolist())
    for blk in live - heads[0] - heads[1] - heads[2]:
        assert w.refcount[blk] == 1
