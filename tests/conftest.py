import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the error figures the parity tests achieved."""
    from helpers import FIGURES
    if not FIGURES:
        return
    terminalreporter.write_sep("-", "parity figures achieved")
    for case, figs in FIGURES:
        terminalreporter.write_line(case + ": " + ", ".join(
            f"{k} {v:.3e}" if isinstance(v, float) else f"{k} {v}" for k, v in figs.items()))
