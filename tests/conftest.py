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
    """The largest attention errors each GPU test saw against the oracle, with the
    output bar of each (1e-2 unless the test derives its own)."""
    gu = sys.modules.get("gpu_util")
    if gu is None or not getattr(gu, "ERRORS", None):
        return
    terminalreporter.write_sep("-", "attention max-abs error against the oracle (out, lse, out bar)")
    for label, (eo, el, bar) in sorted(gu.ERRORS.items()):
        terminalreporter.write_line(f"{eo:.3e}  {el:.3e}  {bar:.1e}  {label}")
    label, (eo, el, bar) = max(gu.ERRORS.items(), key=lambda kv: kv[1][0] / kv[1][2])
    terminalreporter.write_line(f"closest to its bar: out {eo:.3e} of {bar:.1e} ({label}); "
                                f"largest lse error {max(v[1] for v in gu.ERRORS.values()):.3e}; "
                                f"{len(gu.ERRORS)} tests")
