"""The library's block pool (C ABI, host only) against the plain model, and the pages'
accounting and lifecycle invariants ("Capitulo 2", section "Evals deterministas para
esta capa")."""
import numpy as np
import pytest

import paged_kv_cache_27_amd as pkv
from oracle.pool_model import PoolModel


def _state(pool, n):
    return [pool.refcount(i) for i in range(n)]


def _model_state(model, n):
    return [model.ref.get(i, 0) for i in range(n)]


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_match_model(seed):
    """Random allocate / share / release / copy-on-write sequences, including ones that
    must fail (pool exhausted, releasing a free block): after every call the library's
    counts equal the model's, and a failed call changed nothing."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, 40))
    pool, model = pkv.BlockPoolHandle(n), PoolModel(n)
    for _ in range(400):
        op = rng.integers(0, 4)
        held = sorted(model.ref)
        before = _state(pool, n)
        if op == 0:
            k = int(rng.integers(0, n // 2 + 2))
            if k <= model.free_count():
                model.take(pool.alloc(k))
            else:
                with pytest.raises(pkv.PagedKVError) as e:
                    pool.alloc(k)
                assert e.value.status == -7 and _state(pool, n) == before
        elif op == 1:
            ids = rng.choice(n, size=int(rng.integers(1, 4)))
            if model.can_share(ids):
                pool.share(ids)
                model.share(ids)
            else:
                with pytest.raises(pkv.PagedKVError) as e:
                    pool.share(ids)
                assert e.value.status == -8 and _state(pool, n) == before
        elif op == 2:
            ids = rng.choice(held, size=int(rng.integers(1, 4))) if held and rng.random() < 0.8 else \
                rng.choice(n, size=2)
            if model.can_release(ids):
                pool.release(ids)
                model.release(ids)
            else:
                with pytest.raises(pkv.PagedKVError) as e:
                    pool.release(ids)
                assert e.value.status == -8 and _state(pool, n) == before
        elif held:
            b = int(rng.choice(held))
            if model.ref[b] > 1 and model.free_count() == 0:
                with pytest.raises(pkv.PagedKVError) as e:
                    pool.cow(b)
                assert e.value.status == -7 and _state(pool, n) == before
            else:
                got, copied = pool.cow(b)
                model.cow(b, got, copied)
        model.check()
        assert _state(pool, n) == _model_state(model, n)
        assert pool.free_count() == model.free_count()


def test_session_of_32k_tokens_takes_2000_blocks():
    """A 32 K-token session in 16-token blocks holds 2 000 of a 2 800-block pool ("PagedAttention
    por dentro...", section "El pool de bloques"); when it ends they all return."""
    pool = pkv.BlockPoolHandle(2800)
    ids = pool.alloc((32000 + 15) // 16)
    assert ids.size == 2000 and pool.free_count() == 800
    with pytest.raises(pkv.PagedKVError):
        pool.alloc(801)
    pool.release(ids)
    assert pool.free_count() == 2800


def test_beam_fork_copies_only_the_last_block():
    """Four branches share a 45-token prompt (3 blocks).  As each writes its next token,
    copy-on-write copies only the last, partly filled block, and only for the branches
    that still share it; the full blocks stay shared by all four ("PagedAttention por
    dentro...", section "Copy-on-write para sampling paralelo")."""
    pool = pkv.BlockPoolHandle(16)
    table = pool.alloc(3)
    for _ in range(3):
        pool.share(table)
    tables = [table.copy() for _ in range(4)]
    copies = 0
    for t in tables:
        new, copied = pool.cow(int(t[2]))
        copies += copied
        t[2] = new
    assert copies == 3  # the last branch holds the only remaining reference
    assert [pool.refcount(int(b)) for b in table[:2]] == [4, 4]
    assert len({int(t[2]) for t in tables}) == 4
    assert all(pool.refcount(int(t[2])) == 1 for t in tables)
    assert pool.free_count() == 16 - 3 - 3


def test_argument_errors():
    lib = pkv.load_library()
    assert lib.pkv_pool_create(0) is None
    pool = pkv.BlockPoolHandle(4)
    with pytest.raises(pkv.PagedKVError):
        pool.refcount(4)
    with pytest.raises(pkv.PagedKVError):
        pool.cow(1)  # not allocated
    with pytest.raises(pkv.PagedKVError):
        pool.share([-1])
    assert pool.free_count() == 4
