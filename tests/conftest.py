import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a `key v1 v2 ...` fixture (lines starting with # are comments)."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def pytest_terminal_summary(terminalreporter):
    """Parity margins of the run: for every passing tolerance check, its worst
    elementwise error in units of its bound and its relative RMS error in
    units of its tolerance (1.0 = at the bound)."""
    helpers = sys.modules.get("helpers")
    rows = getattr(helpers, "MARGINS", None)
    if not rows:
        return
    tr = terminalreporter
    tr.section("parity margins (fraction of the bound used)")
    worst_by_test = {}
    for test, what, m_el, m_rms in rows:
        k = test or "?"
        w = worst_by_test.get(k)
        if w is None or max(m_el, m_rms) > max(w[1], w[2]):
            worst_by_test[k] = (what, m_el, m_rms)
    for test in sorted(worst_by_test):
        what, m_el, m_rms = worst_by_test[test]
        tr.write_line(f"{m_el:6.3f} elementwise  {m_rms:6.3f} rel-RMS  {test}  [{what}]")
    top = max(max(m_el, m_rms) for _, _, m_el, m_rms in rows)
    tr.write_line(f"{len(rows)} checks; largest fraction of a bound used: {top:.3f}")
