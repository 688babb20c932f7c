"""The fp64 oracle against what the definition and the mathematics fix (CPU only)."""
import pytest

import oracle.fno_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(O)
