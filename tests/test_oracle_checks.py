"""Pins of the input-check oracle (oracle/checks.py), on the CPU.

* hand-worked cases: each rule on a few entries whose answer is read off the rule by
  hand (the expected triples are written out in the comments);
* valid inputs -- the generated workloads' tables, contexts, new-token positions,
  prefix groups, prefill chunks and copy-on-write pairs from a block pool -- break no
  rule;
* one planted violation of each kind in a valid input is found alone, with its code and
  index.
"""
import numpy as np
import pytest

from oracle import checks as C
from workloads import LLAMA8B, PREFIX, make_workload, prefill_queries
from workloads.synth import BlockPool

NONE = (0, C.OK, -1)


def test_slots_by_hand():
    # 4 blocks of 16: rows 0..63.  Slots 64 and -1 are outside (write nothing).
    # Active keys 5 7 5 . 5 . . 63 7 -> duplicates at t = 2, 4, 8.
    assert C.check_slots(np.array([5, 7, 5, -1, 5, 64, 64, 63, 7]), 4, 16) == (3, C.DUPLICATE_SLOT, 2)
    assert C.check_slots(np.array([], np.int64), 4, 16) == NONE
    assert C.check_slots(np.array([64, 64, -5, -5]), 4, 16) == NONE


def test_positions_by_hand():
    bt = np.array([[3, 1], [1, 0]], np.int32)  # 2 sequences, 2 blocks each, B = 16
    seq = [0, 1, 0, 1, 2, -1, 0, 1, 0]
    pos = [0, 16, 17, 1, 0, 5, 40, 0, 0]
    # slots: 48, 0, 17, 17 (dup of t=2), seq 2 >= 2 (SEQ_ID at 4), skip, past the row
    # (skip), 16, 48 (dup of t=0)  ->  3 violations, lowest code 1 at t = 3
    assert C.check_positions(np.array(seq), np.array(pos), 2, bt, 4, 16) == (3, C.DUPLICATE_SLOT, 3)
    assert C.check_positions(np.array([2, 5]), np.array([0, 0]), 2, bt, 4, 16) == (2, C.SEQ_ID, 0)
    # a block ID outside the pool gives a slot outside the cache: no write, no violation
    bt2 = np.array([[9, 9]], np.int32)
    assert C.check_positions(np.array([0, 0]), np.array([3, 3]), 1, bt2, 4, 16) == NONE


def test_decode_by_hand():
    bt = np.array([[4, 5, -1, 9], [0, 0, 0, 0], [7, 7, 7, 7]], np.int32)  # 5 blocks, B = 16
    # s0: 20 tokens read blocks 0, 1 -> entry 1 (ID 5) is outside [0, 5); entries 2, 3 unread
    # s1: 70 > 64 -> CONTEXT_LEN at 1; s2: empty, reads nothing
    assert C.check_decode(bt, np.array([20, 70, 0]), 64, 5, 16) == (2, C.CONTEXT_LEN, 1)
    assert C.check_decode(bt, np.array([20, 64, 0]), 64, 5, 16) == (1, C.BLOCK_ID, 1)
    assert C.check_decode(bt, np.array([-1, 64, 0]), 64, 5, 16) == (1, C.CONTEXT_LEN, 0)


def test_window_reads_only_attended_blocks():
    bt = np.array([[7, 9, 8, 2]], np.int32)  # 5 blocks; IDs 7, 9, 8 are outside
    # 64 tokens, window 20, 1 sink: positions >= 44 or < 1 -> blocks 0, 2, 3 (not 1)
    assert C.check_decode(bt, np.array([64]), 64, 5, 16, window=20, sinks=1) == (2, C.BLOCK_ID, 0)
    assert C.check_decode(bt, np.array([64]), 64, 5, 16) == (3, C.BLOCK_ID, 0)
    # no sink: blocks 2, 3 only
    assert C.check_decode(bt, np.array([64]), 64, 5, 16, window=20) == (1, C.BLOCK_ID, 2)


def _prefix_case():
    bt = np.array([[1, 2, 3, 0, 0], [1, 2, 4, 0, 0], [1, 6, 5, 0, 0], [7, 8, 0, 0, 0], [7, 9, 0, 0, 0]],
                  np.int32)
    return bt, np.array([40, 33, 50, 17, 20]), np.array([0, 3, 5]), np.array([32, 32, 32, 16, 16])


def test_shared_prefix_by_hand():
    bt, ctx, gs, pl = _prefix_case()
    # group 0 = sequences 0-2 sharing 32 tokens (2 blocks of 16): s2's entry 1 (6) differs
    # from s0's (2) -> PREFIX_BLOCKS at 2 * 5 + 1 = 11.  Group 1 = 3-4 sharing 1 block: equal.
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, gs, 3, pl, 32) == (1, C.PREFIX_BLOCKS, 11)
    pl2 = pl.copy()
    pl2[1] = 48  # above max_prefix_len and unequal to the group's 32
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, gs, 3, pl2, 32) == (2, C.PREFIX_LEN, 1)
    pl3 = pl.copy()
    pl3[3] = 8  # not a multiple of B: s3 (and s4, unequal to it) break PREFIX_LEN; the
    #             first's prefix is unusable, so group 1's tables are not compared
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, gs, 3, pl3, 32) == (3, C.PREFIX_LEN, 3)
    pl4 = pl.copy()
    pl4[4] = 32  # 32 > context 20 of s4, and unequal to s3's 16
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, gs, 3, pl4, 32) == (2, C.PREFIX_LEN, 4)


def test_group_starts_by_hand():
    bt, ctx, _, pl = _prefix_case()
    # a group of 4 above max_group_size 3: entry 0; the prefix rules are then skipped
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, np.array([0, 4, 5]), 3, pl, 32) == (1, C.GROUP_STARTS, 0)
    # the last entry must be num_seqs
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, np.array([0, 3, 4]), 3, pl, 32) == (1, C.GROUP_STARTS, 2)
    # decreasing, and an entry past num_seqs
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, np.array([0, 3, 2, 5]), 3, pl, 32) == (1, C.GROUP_STARTS, 1)
    assert C.check_shared_prefix(bt, ctx, 100, 10, 16, np.array([1, 6, 5]), 5, pl, 32) == (2, C.GROUP_STARTS, 0)


def test_prefill_by_hand():
    bt = np.array([[1, 9, 0, 0], [99, 99, 99, 99], [99, 99, 99, 99]], np.int32)  # 8 blocks, B = 16
    # rows 5, 0, 15: s2's 15 > max_q_len 10 (QUERY_ROWS at 2, its blocks not checked);
    # s1 has no rows (reads nothing); s0 reads blocks 0, 1 of 30 tokens: ID 9 at entry 1
    assert C.check_prefill(np.array([0, 5, 5, 20]), 10, bt, np.array([30, 10, 40]), 64, 8, 16) == \
        (2, C.BLOCK_ID, 1)
    # cu_q[0] != 0 breaks s0's rows too
    assert C.check_prefill(np.array([1, 5, 5, 20]), 10, bt, np.array([30, 10, 40]), 64, 8, 16) == \
        (2, C.QUERY_ROWS, 0)
    # more rows than context, and a context past the bound
    assert C.check_prefill(np.array([0, 5, 5, 8]), 10, bt, np.array([4, 10, 70]), 64, 8, 16) == \
        (2, C.CONTEXT_LEN, 2)


def test_block_ids_by_hand():
    # 8 blocks.  Pair 3's source 9 is outside: inactive.  Active sources {1, 2, 3, 4}:
    # pair 1 repeats destination 5, pair 2's destination 2 is a source.
    assert C.check_block_ids(np.array([1, 2, 3, 9, 4]), np.array([5, 5, 2, 6, 7]), 8) == (2, C.BLOCK_PAIR, 1)
    assert C.check_block_ids(np.array([3]), np.array([3]), 8) == (1, C.BLOCK_PAIR, 0)  # onto itself
    # swap in (no sources): repeated IDs only; -1 and 8 are outside
    assert C.check_block_ids(None, np.array([3, 3, -1, 8, 3]), 8) == (2, C.BLOCK_PAIR, 1)
    assert C.check_block_ids(None, np.array([], np.int32), 8) == NONE


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_valid_workloads_break_no_rule(seed):
    w = make_workload(LLAMA8B.replace(num_seqs=12, num_q_heads=8, num_kv_heads=2, ctx_params=(1, 900), seed=seed))
    c = w.cfg
    assert C.check_decode(w.block_tables, w.context_lens, w.max_context_len, w.num_blocks, c.block_size) == NONE
    assert C.check_positions(w.new_seq, w.new_pos, c.num_seqs, w.block_tables, w.num_blocks, c.block_size) == NONE
    assert C.check_positions(w.hist_seq, w.hist_pos, c.num_seqs, w.block_tables, w.num_blocks, c.block_size) == NONE
    slots = [C.resolve_slot(int(s), int(p), w.block_tables, c.block_size) for s, p in zip(w.new_seq, w.new_pos)]
    assert C.check_slots(np.array(slots), w.num_blocks, c.block_size) == NONE
    chunks = np.minimum(w.context_lens, 1 + np.arange(c.num_seqs) * 7)
    _, cu = prefill_queries(w, chunks, seed)
    assert C.check_prefill(cu, int(chunks.max()), w.block_tables, w.context_lens, w.max_context_len, w.num_blocks,
                           c.block_size) == NONE
    # copy-on-write pairs: each shared block copied into a fresh one from the pool
    pool = BlockPool(64, np.random.default_rng(seed))
    held = [pool.allocate() for _ in range(10)]
    shared = [pool.share(b) for b in held[:5]]
    pairs = np.array([(b, pool.allocate()) for b in shared], np.int32)
    assert C.check_block_ids(pairs[:, 0], pairs[:, 1], 64) == NONE
    assert C.check_block_ids(None, pairs[:, 1], 64) == NONE


def test_prefix_workload_breaks_no_rule():
    w = make_workload(PREFIX.replace(num_seqs=24, num_q_heads=8, num_kv_heads=2, ctx_params=(256, 0, 100),
                                     prefix_groups=3, seed=5))
    c = w.cfg
    gs = np.asarray(w.prefix_group_starts(), np.int32)
    pl = np.full(c.num_seqs, 256, np.int32)
    assert C.check_shared_prefix(w.block_tables, w.context_lens, w.max_context_len, w.num_blocks, c.block_size,
                                 gs, int(np.diff(gs).max()), pl, 256) == NONE


def test_planted_violations_are_found_alone():
    w = make_workload(LLAMA8B.replace(num_seqs=10, num_q_heads=8, num_kv_heads=2, ctx_params=(40, 700), seed=9))
    c = w.cfg
    B, mb = c.block_size, w.block_tables.shape[1]
    rng = np.random.default_rng(0)
    for _ in range(20):
        s = int(rng.integers(c.num_seqs))
        j = int(rng.integers(-(-int(w.context_lens[s]) // B)))
        bt = w.block_tables.copy()
        bt[s, j] = w.num_blocks + int(rng.integers(0, 3))
        assert C.check_decode(bt, w.context_lens, w.max_context_len, w.num_blocks, B) == (1, C.BLOCK_ID, s * mb + j)
        ctx = w.context_lens.copy()
        ctx[s] = w.max_context_len + 1
        assert C.check_decode(w.block_tables, ctx, w.max_context_len, w.num_blocks, B) == (1, C.CONTEXT_LEN, s)
        t, u = sorted(int(x) for x in rng.choice(c.num_seqs, 2, replace=False))
        seq, pos = w.new_seq.copy(), w.new_pos.copy()
        seq[u], pos[u] = seq[t], pos[t]  # token u writes token t's slot
        assert C.check_positions(seq, pos, c.num_seqs, w.block_tables, w.num_blocks, B) == (1, C.DUPLICATE_SLOT, u)
