import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes of CPU oracle time)")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    from tests import report
    if report.LINES:
        terminalreporter.write_sep("-", "parity statistics (GPU against the oracle)")
        for line in report.LINES:
            terminalreporter.write_line(line)
