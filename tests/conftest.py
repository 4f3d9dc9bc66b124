import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU oracle run")


def pytest_terminal_summary(terminalreporter):
    """Worst achieved parity error of each test that compared against the oracle, beside
    its gate (output: max-abs error over the RMS per-vector norm |v|; state: relative
    Frobenius error)."""
    try:
        from gdn_testutil import PARITY_LOG, tolerances
    except ImportError:
        return
    if not PARITY_LOG:
        return
    tr = terminalreporter
    tr.write_sep("-", "parity against the float64 oracle (worst unit of each test)")
    tr.write_line(f"{'test':78s} {'dtype':5s} {'units':>5s} {'max|do|/|v|':>11s} {'gate':>7s} {'state rel':>9s} {'gate':>7s}")
    for key in sorted(PARITY_LOG):
        r = PARITY_LOG[key]
        fo, fs = tolerances(r["dtype"])
        eo = "n/a" if r["o"] is None else f"{r['o']:.2e}"
        es = "n/a" if r["s"] is None else f"{r['s']:.2e}"
        tr.write_line(f"{key[-78:]:78s} {r['dtype']:5s} {r['units']:5d} {eo:>11s} {fo:7.0e} {es:>9s} {fs:7.0e}")
