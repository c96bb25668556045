"""The CPU oracle against its pins (golden closed forms, brute force,
invariants).  CPU only."""

import pytest

import oracle.paged_attention as orc
import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(orc)
