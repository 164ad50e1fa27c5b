"""The CPU oracle against its pins (facts fixed by the pages and by
mathematics, never the oracle's own formula retyped)."""
import pytest

from oracle import ref
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(ref)
