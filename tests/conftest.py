import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# (test id, what, max abs error, bar) of the parity checks that report their margin
_MARGINS = []


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: longer CPU test")


@pytest.fixture
def margin(request):
    """margin(what, err, bar): record a parity check's largest error against its bar
    (listed at the end of the run, so the record of a passing run holds the figures)."""
    def record(what: str, err: float, bar: float) -> None:
        _MARGINS.append((request.node.name, what, float(err), float(bar)))
    return record


def pytest_terminal_summary(terminalreporter):
    if not _MARGINS:
        return
    terminalreporter.write_sep("-", "parity margins (max abs error against the bar)")
    for name, what, err, bar in _MARGINS:
        terminalreporter.write_line(f"{name} {what}: {err:.3e} (bar {bar:.0e})")
