"""Debug mode of the binding, on the CPU: with PAGEDKV_DEBUG set, each entry point runs its
input check before anything else and raises PreconditionError when the check reports a
violation; without it (or set to 0) the check is not run.  The checks themselves are
replaced here by stubs that record their calls, so no GPU is needed: a refused call
returns before its tensors are handed to the library, and a call that goes on fails at
once on the CPU tensors (ValueError), which shows the check was skipped."""
import pytest
import torch

import paged_kv_cache_27_amd as pkv
from paged_kv_cache_27_amd import _checks

BAD = pkv.CheckResult(3, 4, 17)


def _i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


CACHE = torch.zeros((8, 2, 16, 64), dtype=torch.bfloat16)
Q = torch.zeros((2, 4, 64), dtype=torch.bfloat16)

# entry point, the check it runs, and a call with CPU tensors of plausible shapes
CALLS = {
    "paged_kv_write": ("paged_kv_check_slots", lambda: pkv.paged_kv_write(
        torch.zeros(2, dtype=torch.int64), Q[:, :2], Q[:, :2], CACHE, CACHE)),
    "paged_kv_write_positions": ("paged_kv_check_positions", lambda: pkv.paged_kv_write_positions(
        _i32(2), _i32(2), _i32(2, 4), Q[:, :2], Q[:, :2], CACHE, CACHE)),
    "paged_attention_decode": ("paged_attention_check_decode", lambda: pkv.paged_attention_decode(
        Q, CACHE, CACHE, _i32(2, 4), _i32(2), 0.125, Q.clone(), 64)),
    "paged_attention_decode_noalloc": ("paged_attention_check_decode", lambda: pkv.paged_attention_decode_noalloc(
        Q, CACHE, CACHE, _i32(2, 4), _i32(2), 0.125, Q.clone(), 64)),
    "paged_attention_decode_window": ("paged_attention_check_decode", lambda: pkv.paged_attention_decode_window(
        Q, CACHE, CACHE, _i32(2, 4), _i32(2), 0.125, Q.clone(), 64, 16, 4)),
    "paged_attention_decode_shared_prefix": (
        "paged_attention_check_shared_prefix", lambda: pkv.paged_attention_decode_shared_prefix(
            Q, CACHE, CACHE, _i32(2, 4), _i32(2), 0.125, Q.clone(), 64, _i32(2), _i32(2), 2, 32)),
    "paged_attention_prefill": ("paged_attention_check_prefill", lambda: pkv.paged_attention_prefill(
        Q, _i32(3), 1, CACHE, CACHE, _i32(2, 4), _i32(2), 0.125, Q.clone(), 64)),
    "paged_kv_copy_blocks": ("paged_kv_check_block_ids", lambda: pkv.paged_kv_copy_blocks(
        _i32(2), _i32(2), CACHE, CACHE)),
    "paged_kv_swap_in": ("paged_kv_check_block_ids", lambda: pkv.paged_kv_swap_in(
        _i32(2), CACHE[:2].clone(), CACHE[:2].clone(), CACHE, CACHE)),
}


@pytest.fixture
def stubs(monkeypatch):
    seen = []
    for name in {c for c, _ in CALLS.values()}:
        monkeypatch.setattr(_checks, name, lambda *a, _n=name, **k: (seen.append(_n), BAD)[1])
    return seen


@pytest.mark.parametrize("fn", sorted(CALLS))
def test_debug_mode_refuses_before_launching(fn, stubs, monkeypatch):
    check, call = CALLS[fn]
    monkeypatch.setenv("PAGEDKV_DEBUG", "1")
    with pytest.raises(pkv.PreconditionError) as e:
        call()
    assert e.value.result == BAD
    assert stubs == [check]
    assert fn in str(e.value) and "block ID at index 17" in str(e.value)


@pytest.mark.parametrize("value", [None, "0"])
@pytest.mark.parametrize("fn", sorted(CALLS))
def test_without_debug_mode_no_check_runs(fn, value, stubs, monkeypatch):
    if value is None:
        monkeypatch.delenv("PAGEDKV_DEBUG", raising=False)
    else:
        monkeypatch.setenv("PAGEDKV_DEBUG", value)
    with pytest.raises((ValueError, AssertionError)):  # the CPU tensors are refused at once
        CALLS[fn][1]()
    assert stubs == []


def test_clean_check_lets_the_call_through(monkeypatch):
    monkeypatch.setenv("PAGEDKV_DEBUG", "1")
    monkeypatch.setattr(_checks, "paged_kv_check_slots", lambda *a, **k: pkv.CheckResult(0, 0, -1))
    with pytest.raises(ValueError):  # past the check, the CPU tensors are refused
        CALLS["paged_kv_write"][1]()
