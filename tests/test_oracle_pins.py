"""The CPU oracle against brute force, library routines, invariants and the
figures printed on the pages (no GPU needed)."""
import pytest

import oracle_checks as C


@pytest.mark.parametrize("check", C.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
