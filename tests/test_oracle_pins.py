"""The CPU oracle pinned to the pages' printed values, closed forms, brute force and independent library routines."""
import pytest

from tests import oracle_checks as C


@pytest.mark.parametrize("check", C.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
