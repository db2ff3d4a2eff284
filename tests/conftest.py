import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
for _p in (ROOT, HERE):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libdg.so")
    config.addinivalue_line("markers", "slow: full-size workload (seconds of CPU work)")


GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_terminal_summary(terminalreporter):
    """Max err/bound per parity case: the full-size workloads and the ten
    cases closest to the bound."""
    import parity_log
    rows = parity_log.RATIOS
    tr = terminalreporter
    for n in parity_log.NOTES:
        tr.write_line(n)
    if not rows:
        return
    full = [r for r in rows if r[0].startswith("workload")]
    worst = sorted(rows, key=lambda r: -r[1])[:10]
    tr.write_line(f"parity: {len(rows)} comparisons, max err/bound {max(r[1] for r in rows):.3g}")
    for name, ratio in full + [r for r in worst if r not in full]:
        tr.write_line(f"  {ratio:8.3g}  {name}")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN
