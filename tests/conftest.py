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
    import margins
    if not margins.RECORDS:
        return
    terminalreporter.write_sep("-", "parity margins (max |out - ref| / max |ref|)")
    for name, err, tol in margins.RECORDS:
        terminalreporter.write_line(f"{name}: err {err:.3e} tol {tol:.0e} ({100 * err / tol:.1f}% of tol)")
