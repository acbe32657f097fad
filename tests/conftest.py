import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

_CONFIG = None


def pytest_configure(config):
    global _CONFIG
    _CONFIG = config
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_runtest_logreport(report):
    """Echo the margins each parity check printed ("[parity] ..." lines) to
    the terminal even when output is captured, so every run's log records the
    headroom left under each tolerance."""
    if report.when != "call" or not report.passed or _CONFIG is None:
        return
    lines = [l for l in report.capstdout.splitlines() if "[parity]" in l]
    tr = _CONFIG.pluginmanager.get_plugin("terminalreporter")
    if not lines or tr is None:
        return
    tr.write_line("")
    tr.write_line(f"{report.nodeid}:")
    for l in lines:
        tr.write_line("    " + l.strip())


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
