import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Per-tensor parity table of the GPU comparisons (printed also under -q)."""
    gu = sys.modules.get("gpu_util")
    if gu is not None and getattr(gu, "RESULTS", None):
        gu.write_summary(terminalreporter.write_line)
