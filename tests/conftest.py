import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Largest error against the oracle of each GPU comparison, so the margin
    under the tolerance is visible even in a quiet run."""
    gc = sys.modules.get("gpu_common")
    if gc is None or not gc.ERRORS:
        return
    worst = {}
    for what, dtype, err, tol in gc.ERRORS:
        key = (what, dtype)
        if key not in worst or err > worst[key][0]:
            worst[key] = (err, tol)
    terminalreporter.section("max abs error against the oracle")
    for (what, dtype), (err, tol) in sorted(worst.items(), key=lambda x: -x[1][0] / x[1][1]):
        terminalreporter.write_line(f"{err:10.3e}  ({100 * err / tol:5.1f}% of {tol:.0e})  {dtype:4s}  {what}")
