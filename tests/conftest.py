import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """Largest parity errors the GPU tests measured, per quantity and verify form."""
    gh = sys.modules.get("gpu_harness")
    if gh is None or not gh.MAX_ERR:
        return
    terminalreporter.write_sep("-", "largest parity errors measured (quantity, verify form)")
    for (what, mode), err in sorted(gh.MAX_ERR.items()):
        terminalreporter.write_line(f"{what:>10s} {mode:>6s}  {err:.3e}")
