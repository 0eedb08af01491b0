"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
from oracle_pins import CHECKS


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(orc, check):
    check(orc)
