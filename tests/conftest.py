import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU work (full-size oracle samples)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """The largest attention errors each GPU test saw against the oracle (bar 1e-2)."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not getattr(gu, "ERRORS", None):
        return
    terminalreporter.write_sep("-", "attention max-abs error against the oracle (out, lse)")
    for label, (eo, el) in sorted(gu.ERRORS.items()):
        terminalreporter.write_line(f"{eo:.3e}  {el:.3e}  {label}")
    worst = max(max(v) for v in gu.ERRORS.values())
    terminalreporter.write_line(f"worst {worst:.3e} over {len(gu.ERRORS)} tests")
