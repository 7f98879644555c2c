import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The largest err/bound of every full-size parity check that ran."""
    try:
        from tests import gpu_util
    except Exception:
        return
    if not gpu_util.REPORT:
        return
    terminalreporter.section("largest err/bound per workload")
    for name, worst in gpu_util.REPORT:
        terminalreporter.write_line(f"{name}: {worst:.3g}")
