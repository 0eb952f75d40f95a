import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


# Parity figures: what the passing GPU tests print (index-agreement fractions,
# error ratios against their bounds) is collected and repeated at the end of
# the run, so that a quiet (-q) log still carries the measured numbers.
_FIGURES = []


@pytest.hookimpl(hookwrapper=True)
def pytest_runtest_makereport(item, call):
    outcome = yield
    rep = outcome.get_result()
    if rep.when == "call" and rep.passed and item.get_closest_marker("gpu") is not None:
        out = rep.capstdout.strip()
        if out:
            _FIGURES.append((item.nodeid, out))


def pytest_terminal_summary(terminalreporter):
    if not _FIGURES:
        return
    tr = terminalreporter
    tr.section("parity figures (stdout of the passing GPU tests)")
    for nodeid, out in _FIGURES:
        tr.write_line(nodeid)
        for line in out.splitlines():
            tr.write_line("    " + line)
