import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    oracle.build()
    return oracle


def pytest_terminal_summary(terminalreporter):
    cases = sys.modules.get("gpu_cases")
    log = getattr(cases, "PARITY_LOG", None)
    if log:
        terminalreporter.write_sep("-", "whole-output parity (max abs error vs the fp64 oracle)")
        for what, err, tol in log:
            terminalreporter.write_line(f"{what}: {err:.3e} (tolerance {tol:g})")
