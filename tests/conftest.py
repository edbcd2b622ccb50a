import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """Rows compared, exact and flagged (explained by a bf16 rounding the fp32
    accumulation bound allows) of every top-k / tail acceptance run."""
    from tests import helpers
    if helpers.PARITY_COUNTS:
        terminalreporter.section("top-k / tail parity counts")
        for what, rows, exact, flagged in helpers.PARITY_COUNTS:
            terminalreporter.write_line(f"{what}: rows {rows} exact {exact} flagged {flagged}")
