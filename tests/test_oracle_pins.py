"""The CPU oracle against facts fixed by the pages and by mathematics."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.default())
