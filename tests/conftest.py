import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.load()


def pytest_terminal_summary(terminalreporter):
    """fp32 dG elements that met the 1e-5 bar only under the cancellation
    scale (dT_g/dG's two terms cancelling by >= 100x): reported, expected 0."""
    cmp = sys.modules.get("compare")
    tally = getattr(cmp, "RELAXED_TALLY", None)
    if tally and tally["checked"]:
        terminalreporter.write_line(
            f"fp32 dG: {tally['relaxed']} of {tally['checked']} elements within the bar only under the "
            f"cancellation scale")
