"""The CPU oracle against the pages' worked examples, closed forms, a library routine,
brute-force recurrences and invariants (the pins live in oracle_pins.py)."""
import pytest

import oracle_pins
from oracle import attention as att
from oracle import online as onl


@pytest.mark.parametrize("name", sorted(oracle_pins.PINS))
def test_pin(name):
    oracle_pins.PINS[name](att, onl)


def test_page_arithmetic():
    """The page's size figures follow from their shapes (used as context only)."""
    g = oracle_pins.GOLDEN["score_matrix_bytes"]
    assert g["N"] ** 2 * g["bytes_per_element"] == g["printed_MiB"] * 2 ** 20
    t = oracle_pins.GOLDEN["tile_count"]
    assert t["N"] ** 2 == t["printed_pairs"]
    assert t["tile"] ** 2 == t["printed_tile_slots"]
    assert t["printed_pairs"] // t["printed_tile_slots"] == 4096
