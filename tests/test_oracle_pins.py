"""The CPU oracle against facts fixed outside it (closed forms, invariants,
exact brute force, library routines).  See tests/pins.py for each source."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_golden_table_is_current():
    """The stored closed-form table is what its generator writes today."""
    import os
    import subprocess
    import sys

    golden = pins.GOLDEN
    before = open(golden).read()
    subprocess.run([sys.executable, os.path.join(os.path.dirname(golden), "make_constant_rows.py")],
                   check=True, capture_output=True)
    assert open(golden).read() == before
