import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def pytest_terminal_summary(terminalreporter):
    """The output checks' errors (whole tensor and worst row) in the run's
    log, also when pytest captures the tests' own output."""
    helpers = sys.modules.get("helpers")   # the module the tests imported
    PARITY_LOG = getattr(helpers, "PARITY_LOG", None)
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.section("output parity against the oracle (relative L2)")
    for label, whole, worst, row, n, tol in PARITY_LOG:
        tr.write_line(f"{label}: whole {whole:.2e}, worst row {worst:.2e} (row {row} of {n}), tolerance {tol:g}")
