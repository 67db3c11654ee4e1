"""The CPU oracle against facts fixed outside it (closed forms, invariants,
exact brute force, library routines).  See tests/pins.py for each source."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


def test_golden_table_is_current(tmp_path):
    """The stored closed-form table is what its generator writes today (written
    to a temporary file: the committed table is never rewritten by a test)."""
    import os
    import subprocess
    import sys

    golden = pins.GOLDEN
    fresh = tmp_path / "constant_rows.txt"
    subprocess.run([sys.executable, os.path.join(os.path.dirname(golden), "make_constant_rows.py"), str(fresh)],
                   check=True, capture_output=True)
    assert fresh.read_text() == open(golden).read()
