import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


_CONFIG = None


def pytest_configure(config):
    global _CONFIG
    _CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU case")


def progress(line):
    """Write a line to the terminal at once, also while pytest captures the test's output (the
    full-size checks run minutes of oracle work per test, and a run that prints nothing for
    minutes looks hung)."""
    tr = _CONFIG.pluginmanager.getplugin("terminalreporter") if _CONFIG else None
    capman = _CONFIG.pluginmanager.getplugin("capturemanager") if _CONFIG else None
    if tr is None or capman is None:
        print(line, flush=True)
        return
    with capman.global_and_fixture_disabled():
        tr.write_line(line)
        tw = getattr(tr, "_tw", None)  # the reporter's terminal writer, flushed when present
        if tw is not None:
            tw.flush()


def pytest_terminal_summary(terminalreporter):
    """Near-tie accounting of the parity checks that ran, shown also under -q."""
    mod = sys.modules.get("parity_util")
    lines = getattr(mod, "REPORT", None) if mod else None
    if lines:
        terminalreporter.section("near-tie accounting")
        for line in lines:
            terminalreporter.write_line(line)
