"""The oracle against what the pages and mathematics fix (CPU only)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name, oracle_lib):
    ALL_PINS[name](oracle_lib)
