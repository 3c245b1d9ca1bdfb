import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Raw O / LSE errors of every parity check of the run."""
    try:
        from parity_checks import REPORT
    except ImportError:
        return
    if REPORT:
        terminalreporter.section("parity: raw errors against the oracle")
        for line in REPORT:
            terminalreporter.write_line(line)
