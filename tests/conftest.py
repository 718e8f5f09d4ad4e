import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running")


def pytest_terminal_summary(terminalreporter):
    import errlog
    if not errlog.RECORDS:
        return
    tr = terminalreporter
    tr.section("measured errors (max|y - y_ref| / max|y_ref| unless noted)")
    for case, err, bar in errlog.RECORDS:
        tr.write_line("%-48s %.3e  (bar %.1e)" % (case, err, bar))
