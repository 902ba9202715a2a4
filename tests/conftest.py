import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


def pytest_terminal_summary(terminalreporter):
    """Near-tie accounting of the parity checks that ran, shown also under -q."""
    mod = sys.modules.get("parity_util")
    lines = getattr(mod, "REPORT", None) if mod else None
    if lines:
        terminalreporter.section("near-tie accounting")
        for line in lines:
            terminalreporter.write_line(line)
