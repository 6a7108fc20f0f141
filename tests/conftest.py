import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Print every parity comparison of the session (max |gpu - oracle| per
    compared output, with its bar), so a quiet run of passing GPU tests still
    records the figures."""
    util = sys.modules.get("tests.fa_gpu_util")
    lines = getattr(util, "PARITY_LINES", None) if util else None
    if lines:
        terminalreporter.section("parity: max |gpu - oracle| per comparison")
        for line in lines:
            terminalreporter.write_line(line)
