import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


_WORKLOADS = {}


@pytest.fixture(scope="session")
def workload_cache():
    """Seeded host inputs of the named full-size workload, generated once."""
    from fmha_fwd_amd import workloads as W

    def get(name):
        if name not in _WORKLOADS:
            _WORKLOADS.clear()  # keep one full-size workload in memory at a time
            _WORKLOADS[name] = W.generate(W.SPECS[name])
        return _WORKLOADS[name]
    return get


def pytest_terminal_summary(terminalreporter):
    """Counts of the parity comparisons run in this session: elements compared,
    one-ulp differences, and elements over the max-abs bar excused by the
    oracle's P-rounding bound (with the cap each comparison was held to)."""
    try:
        import harness
    except ImportError:
        return
    if not harness.RECORDS:
        return
    tw = terminalreporter
    tw.section("parity counts")
    n = sum(r["n"] for _, r in harness.RECORDS)
    ties = sum(r["n_tie"] for _, r in harness.RECORDS)
    ulps = sum(r["n_ulp"] for _, r in harness.RECORDS)
    tw.line(f"{len(harness.RECORDS)} comparisons, {n} elements, {ulps} one-ulp differences, "
            f"{ties} excused by the P-rounding bound (fraction {ties / max(n, 1):.2e})")
    worst = sorted(harness.RECORDS, key=lambda wr: -wr[1]["n_tie"] / max(wr[1]["n"], 1))[:8]
    for what, r in worst:
        tw.line(f"  {what}: n={r['n']} n_tie={r['n_tie']} (cap {r['tie_cap']}, oracle candidates {r['n_cand']}) "
                f"n_ulp={r['n_ulp']} "
                f"maxabs={r['maxabs']:.3e} cos={r['cos']:.7f}")
