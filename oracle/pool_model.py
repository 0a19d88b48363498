"""Plain model of the block pool's bookkeeping (TEST INFRASTRUCTURE ONLY).

Loaded only by the test suite.  It shares nothing with the library and keeps the
state the pages describe, as a dict: a block is free or held with a reference count.

  * allocation hands out free blocks with count 1 ("PagedAttention por dentro...",
    section "El pool de bloques": one pool shared by every session, blocks taken on
    demand);
  * sharing adds a reference (section "Copy-on-write para sampling paralelo": the
    branches point their tables at the same physical blocks; "La despensa por
    casilleros", section "Prefix caching...": a new request's table points at the
    block that already holds the same prefix);
  * release drops one, and a block with no reference left is free again (section
    "Estrategia 1: recompute" / "Estrategia 2: swap": an evicted or finished
    session's blocks return to the pool);
  * copy-on-write gives the writer a private block: the same block when it holds the
    only reference, else a fresh one (the old block keeps its other references).

Which free block an allocation returns is not fixed by the pages, so the model does
not pick: it checks that the block the library returned was free and records it.
The accounting invariants ("Capitulo 2", section "Evals deterministas para esta
capa": free + allocated = pool; every referenced block allocated) are check().
"""
from __future__ import annotations


class PoolModel:
    def __init__(self, num_blocks: int):
        self.n = num_blocks
        self.ref = {}  # block id -> reference count (>= 1); absent = free

    def free_count(self) -> int:
        return self.n - len(self.ref)

    def take(self, ids) -> None:
        """Record an allocation that returned `ids`: each must have been free."""
        ids = [int(i) for i in ids]
        assert len(ids) <= self.free_count(), "more blocks handed out than were free"
        assert len(set(ids)) == len(ids), "one block handed out twice"
        for i in ids:
            assert 0 <= i < self.n and i not in self.ref, f"block {i} handed out while not free"
            self.ref[i] = 1

    def can_share(self, ids) -> bool:
        return all(int(i) in self.ref for i in ids)

    def share(self, ids) -> None:
        for i in ids:
            self.ref[int(i)] += 1

    def can_release(self, ids) -> bool:
        need = {}
        for i in ids:
            need[int(i)] = need.get(int(i), 0) + 1
        return all(self.ref.get(i, 0) >= k for i, k in need.items())

    def release(self, ids) -> None:
        for i in ids:
            i = int(i)
            self.ref[i] -= 1
            if self.ref[i] == 0:
                del self.ref[i]

    def cow(self, block: int, returned: int, copied: bool) -> None:
        """Record a copy-on-write of `block` that returned (returned, copied)."""
        block = int(block)
        if self.ref[block] == 1:
            assert returned == block and not copied, "a private block must be written in place"
            return
        assert copied, "a shared block must be copied before writing"
        self.take([returned])
        self.ref[block] -= 1

    def check(self) -> None:
        assert self.free_count() + len(self.ref) == self.n
        assert all(c >= 1 for c in self.ref.values())
