import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a gfx950 (MI355X) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


def pytest_terminal_summary(terminalreporter):
    gu = sys.modules.get("gpu_util")
    if gu is not None and gu.WORST["checks"]:
        terminalreporter.write_line(
            f"largest normwise state error over {gu.WORST['checks']} GPU parity checks: "
            f"{gu.WORST['state']:.3e} (bound 1e-5)")
    if gu is not None and gu.WORST["dist_checks"]:
        terminalreporter.write_line(
            f"largest relative MDS distance error over {gu.WORST['dist_checks']} maps: "
            f"{gu.WORST['dist']:.3e} (bound 1e-4)")
    if gu is not None and gu.WORST_BY_TEST:
        terminalreporter.write_line("largest error per test (kind, test, error):")
        for (kind, test), err in sorted(gu.WORST_BY_TEST.items()):
            terminalreporter.write_line(f"  {kind:5s} {test} {err:.3e}")
