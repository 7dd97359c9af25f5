import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


@pytest.fixture(scope="session")
def pins():
    with open(os.path.join(ROOT, "tests", "golden", "capstone_pins.json")) as f:
        return {k: v["value"] for k, v in json.load(f).items() if not k.startswith("_")}


def pytest_terminal_summary(terminalreporter):
    """Per tensor: the verbatim max |d|/(|ref|+1e-6), how many elements only
    the one-ulp clause (B) or only the cancellation floor (C) admitted."""
    try:
        from parity import REPORT
    except ImportError:
        return
    if not REPORT:
        return
    tr = terminalreporter
    tr.section("parity report (verbatim max metric; elements admitted via B / via C)")
    for what, tol, fmt, cancel, n, verb, vb, vc, cos, fails in REPORT:
        tr.write_line(f"{what[:60]:60s} tol {tol:.0e} {str(fmt):5s} n {n:>10d} verbatim {verb:9.2e} "
                      f"B {vb:>7d} C {vc:>7d}{'' if cancel else ' (no C)'} cos {cos:.9f}"
                      f"{'  FAIL ' + str(fails) if fails else ''}")
