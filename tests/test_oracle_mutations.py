"""Each plausible mistake planted in the oracle (on the CPU) breaks at least one pin.

Mutations (see the MUT() sites in oracle/oracle.c):
 1 query head -> KV head as h % H_kv      5 V cache written from K
 2 scores taken against the V cache       6 context short by one token (new token dropped)
 3 block index and offset swapped         7 fp8 encode truncates instead of RNE
 4 softmax scale dropped                  8 bf16 decoded with the wrong shift
 9 window start off by one                10 sink tokens left out of a window
11 copy-on-write copies K into the V cache     12 prefill query misses its own token
"""
import pytest

import pins
from oracle.oracle import Oracle, build

EXPECTED = {
    1: "pin_gqa_head_mapping", 2: "pin_dense_equivalence", 3: "pin_block_addressing_golden",
    4: "pin_dense_equivalence", 5: "pin_write_placement", 6: "pin_ctx1_returns_new_value",
    7: "pin_fp8_codec", 8: "pin_half_codecs", 9: "pin_window_one_is_last_value",
    10: "pin_window_dense", 11: "pin_copy_blocks", 12: "pin_prefill_one_token_is_decode",
}


@pytest.mark.parametrize("mutation", sorted(EXPECTED))
def test_mutation_is_caught(tmp_path, mutation):
    lib = build(tmp_path / f"liboracle_m{mutation}.so", mutation=mutation)
    orc = Oracle(lib)
    assert orc.mutation == mutation
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert EXPECTED[mutation] in failed, (mutation, failed)
