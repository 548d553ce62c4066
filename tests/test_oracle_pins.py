"""The CPU oracle against its pins (library routines, closed forms, brute force,
invariants and the pages' printed numbers). CPU only."""
import pytest

import oracle_pins as P
from oracle import dflash_oracle as O


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(O)
