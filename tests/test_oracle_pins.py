"""The CPU oracle against facts outside itself (see tests/oracle_pins.py)."""
import pytest

import oracle
import oracle_pins as P  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _built_oracle():
    oracle.build(force=False)


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
