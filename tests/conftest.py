import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line per named workload compared against the oracle: rows, exact
    rows, near-tie rows by class (K boundary / order inside the K / group
    boundary) and failures, and whether the strict rule (near ties at the K
    boundary only) holds."""
    try:
        from parity_check import REPORTS
    except Exception:
        return
    if not REPORTS:
        return
    tr = terminalreporter
    tr.write_sep("=", "oracle parity by workload")
    lines = []
    for label, rep in REPORTS:
        line = (f"{label}: rows={rep.rows} exact={rep.exact} near_tie_k={rep.near_tie_k} "
                f"near_tie_order={rep.near_tie_order} near_tie_group={rep.near_tie_group} "
                f"failures={len(rep.failures)} strict={'ok' if rep.strict_ok else 'NO'}")
        lines.append(line)
        tr.write_line(line)
    out = os.environ.get("MOE_ROUTE_PARITY_OUT")  # optional copy of these lines
    if out:
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
