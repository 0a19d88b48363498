"""Plain model of the input checks: which entries of a call's index arrays break the
preconditions the calls leave unchecked on the device (TEST INFRASTRUCTURE ONLY).

Loaded only by the test suite.  It shares nothing with the library.  Every function
walks the entries one by one in Python and lists each violation as (code, index); the
result is (number of violations, lowest code, lowest index with that code), or
(0, 0, -1) when there is none.  The rules are those stated for each check in the
library's header; the preconditions behind them come from the pages:

  * a slot names one cache row, block_tables[s][p / B] * B + p % B ("Optimizacion de
    Inferencia LLM", section "PagedAttention: Conceptos de SO...", get_physical_block),
    and two tokens writing one row in the same call race (DUPLICATE_SLOT);
  * a decode reads the physical block of every logical block holding an attended token
    ("PagedAttention por dentro...", section "La tabla de paginas (block table)";
    section "Sliding window attention": only the window's blocks stay live; section
    "StreamingLLM...": plus the sink tokens), so those IDs must name blocks of the pool
    (BLOCK_ID), and a context cannot be longer than the bound the grid is sized for
    (CONTEXT_LEN);
  * sequences sharing a prefix point their tables at the same blocks ("La despensa por
    casilleros", section "Prefix caching: compartir casilleros con copy-on-write";
    "PagedAttention por dentro...", section "Prefix caching cross-session"): the group
    structure, prefix lengths and shared entries (GROUP_STARTS, PREFIX_LEN,
    PREFIX_BLOCKS);
  * a prefill chunk is the last n_s tokens of its context ("PagedAttention por
    dentro...", section "Chunked prefill integrado con paged KV") (QUERY_ROWS);
  * copy-on-write copies into a fresh block (section "Copy-on-write para sampling
    paralelo"), and a swapped-in block receives one row (section "Estrategia 2: swap")
    (BLOCK_PAIR).
"""
from __future__ import annotations

import numpy as np

OK, DUPLICATE_SLOT, SEQ_ID, CONTEXT_LEN, BLOCK_ID = 0, 1, 2, 3, 4
GROUP_STARTS, PREFIX_LEN, PREFIX_BLOCKS, QUERY_ROWS, BLOCK_PAIR = 5, 6, 7, 8, 9


def _result(found):
    """(violations, code, index) from a list of (code, index) pairs."""
    if not found:
        return (0, OK, -1)
    code = min(c for c, _ in found)
    return (len(found), code, min(i for c, i in found if c == code))


def _duplicates(keys):
    """Positions t whose key (None = inactive) equals the key of an earlier position."""
    seen, out = set(), []
    for t, k in enumerate(keys):
        if k is None:
            continue
        if k in seen:
            out.append(t)
        seen.add(k)
    return out


def check_slots(slot_mapping, num_blocks: int, block_size: int):
    rows = num_blocks * block_size
    keys = [int(x) if 0 <= int(x) < rows else None for x in np.asarray(slot_mapping).reshape(-1)]
    return _result([(DUPLICATE_SLOT, t) for t in _duplicates(keys)])


def resolve_slot(s: int, p: int, block_tables, block_size: int) -> int:
    """The slot of position p of sequence s, -1 when the rule gives none (a negative
    sequence or position, or a block index past the table's row)."""
    if s < 0 or p < 0:
        return -1
    j = p // block_size
    if j >= block_tables.shape[1]:
        return -1
    return int(block_tables[s, j]) * block_size + p % block_size


def check_positions(seq_ids, positions, num_seqs: int, block_tables, num_blocks: int, block_size: int):
    bt = np.asarray(block_tables).reshape(num_seqs, -1) if num_seqs else np.zeros((0, 1), np.int32)
    rows = num_blocks * block_size
    found, keys = [], []
    for t, (s, p) in enumerate(zip(np.asarray(seq_ids).tolist(), np.asarray(positions).tolist())):
        if s >= num_seqs:
            found.append((SEQ_ID, t))
            keys.append(None)
            continue
        slot = resolve_slot(s, p, bt, block_size)
        keys.append(slot if 0 <= slot < rows else None)
    found += [(DUPLICATE_SLOT, t) for t in _duplicates(keys)]
    return _result(found)


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _read_blocks(ctx: int, block_size: int, window: int = 0, sinks: int = 0):
    """Logical blocks holding a token the decode attends to."""
    if window <= 0:
        return list(range(_ceil_div(ctx, block_size)))
    keep = [t for t in range(ctx) if t >= ctx - window or t < sinks]
    return sorted({t // block_size for t in keep})


def _context_and_blocks(found, block_tables, context_lens, max_context_len, num_blocks, block_size,
                        window=0, sinks=0, reads=None):
    """CONTEXT_LEN for every sequence; BLOCK_ID over the entries read by the sequences
    with a valid length for which reads(s) is true (all of them by default)."""
    bt = np.asarray(block_tables)
    mb = bt.shape[1]
    for s, ctx in enumerate(np.asarray(context_lens).tolist()):
        if ctx < 0 or ctx > max_context_len:
            found.append((CONTEXT_LEN, s))
            continue
        if reads is not None and not reads(s):
            continue
        for j in _read_blocks(ctx, block_size, window, sinks):
            if not 0 <= int(bt[s, j]) < num_blocks:
                found.append((BLOCK_ID, s * mb + j))


def check_decode(block_tables, context_lens, max_context_len: int, num_blocks: int, block_size: int,
                 window: int = 0, sinks: int = 0):
    found = []
    _context_and_blocks(found, block_tables, context_lens, max_context_len, num_blocks, block_size, window, sinks)
    return _result(found)


def check_shared_prefix(block_tables, context_lens, max_context_len: int, num_blocks: int, block_size: int,
                        group_starts, max_group_size: int, prefix_lens, max_prefix_len: int):
    found = []
    _context_and_blocks(found, block_tables, context_lens, max_context_len, num_blocks, block_size)
    bt = np.asarray(block_tables)
    mb = bt.shape[1]
    ctx = np.asarray(context_lens).tolist()
    n = len(ctx)
    gs = np.asarray(group_starts).tolist()
    ng = len(gs) - 1
    bad_groups = False
    for j, a in enumerate(gs):
        bad = a < 0 or a > n or (j == 0 and a != 0) or (j == ng and a != n)
        if j < ng:
            size = gs[j + 1] - a
            bad = bad or size < 0 or size > max_group_size
        if bad:
            found.append((GROUP_STARTS, j))
            bad_groups = True
    if not bad_groups:
        pl = np.asarray(prefix_lens).tolist()
        for j in range(ng):
            f = gs[j]
            p0 = pl[f] if gs[j + 1] > f else 0
            first_ok = p0 >= 0 and p0 % block_size == 0 and p0 <= max_prefix_len
            for s in range(gs[j], gs[j + 1]):
                p = pl[s]
                if p < 0 or p % block_size or p > max_prefix_len or p > ctx[s] or p != p0:
                    found.append((PREFIX_LEN, s))
                if s != f and first_ok:
                    for b in range(p0 // block_size):
                        if int(bt[s, b]) != int(bt[f, b]):
                            found.append((PREFIX_BLOCKS, s * mb + b))
    return _result(found)


def check_prefill(cu_q, max_q_len: int, block_tables, context_lens, max_context_len: int, num_blocks: int,
                  block_size: int):
    found = []
    cu = np.asarray(cu_q).tolist()
    ctx = np.asarray(context_lens).tolist()
    rows_ok = []
    for s in range(len(ctx)):
        ns = cu[s + 1] - cu[s]
        bad = (s == 0 and cu[0] != 0) or ns < 0 or ns > max_q_len or ns > ctx[s]
        if bad:
            found.append((QUERY_ROWS, s))
        rows_ok.append(not bad and ns >= 1)
    _context_and_blocks(found, block_tables, context_lens, max_context_len, num_blocks, block_size,
                        reads=lambda s: rows_ok[s])
    return _result(found)


def check_block_ids(src_ids, dst_ids, num_blocks: int):
    dst = np.asarray(dst_ids).tolist()
    src = None if src_ids is None else np.asarray(src_ids).tolist()

    def active(i):
        return 0 <= dst[i] < num_blocks and (src is None or 0 <= src[i] < num_blocks)

    live = [i for i in range(len(dst)) if active(i)]
    sources = {src[i] for i in live} if src is not None else set()
    found, seen = [], set()
    for i in live:
        if dst[i] in seen or dst[i] in sources:
            found.append((BLOCK_PAIR, i))
        seen.add(dst[i])
    return _result(found)
