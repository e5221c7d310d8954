import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Worst per-unit errors of the parity tests, printed at the end of the run so
# that the achieved margins are kept in the run's log even without -s or -rA.
MARGINS = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")


@pytest.fixture
def margin(request):
    """margin(label, value, bar): record one achieved error against its bar."""
    def rec(label, value, bar):
        MARGINS.append((request.node.name, label, float(value), float(bar)))
    return rec


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    if not MARGINS:
        return
    terminalreporter.write_line("parity margins (worst unit, achieved / bar):")
    for name, label, val, bar in MARGINS:
        terminalreporter.write_line(f"  {name} {label}: {val:.3e} / {bar:.0e}")
