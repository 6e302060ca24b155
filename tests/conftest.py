import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds on the CPU")


def read_golden(name):
    """Non-comment, non-blank lines of a golden fixture, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---- measured parity errors, printed at the end of the run ----
# Each GPU parity helper records (case, quantity, error, tolerance); the
# terminal summary lists them, the cases at the benchmark shapes last.
_PARITY = []


def record_parity(case, quantity, err, tol):
    _PARITY.append((str(case), str(quantity), float(err), float(tol)))


def pytest_terminal_summary(terminalreporter):
    if not _PARITY:
        return
    tw = terminalreporter
    tw.write_line("")
    tw.write_line(f"measured parity errors ({len(_PARITY)} comparisons; error / tolerance):")
    whole = [p for p in _PARITY if "whole" in p[0]]
    rest = [p for p in _PARITY if "whole" not in p[0]]
    for case, q, e, t in sorted(rest, key=lambda p: -p[2] / p[3])[:12]:
        tw.write_line(f"  {case}: {q} {e:.2e} / {t:.0e}")
    if len(rest) > 12:
        tw.write_line(f"  ... {len(rest) - 12} more, all at most {max(p[2] / p[3] for p in rest[12:]):.3f} of "
                      f"their tolerance")
    for case, q, e, t in whole:
        tw.write_line(f"  {case}: {q} {e:.2e} / {t:.0e}")
    worst = max(_PARITY, key=lambda p: p[2] / p[3])
    tw.write_line(f"worst ratio {worst[2] / worst[3]:.3f} ({worst[0]}, {worst[1]})")
