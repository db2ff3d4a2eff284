"""The tile-choice overrides (DG_FORCE_TILE: 512 / 256 = one tile shape for
every problem, 3256 = the shared-B 256 x 256 tile for every dense problem,
8256 /
4128 / 264 = one narrow tile wherever a narrow tile is used; DG_TAIL_TILE:
0 = no separate last round, 8256 / 4128 / 264 = that narrow tile for it; DG_SPLITK:
1 = never split K, S = split every tiled launch S ways) give
results inside the parity bound.  The library reads them once per process, so every setting
runs tests/override_child.py in a child process.  Needs a GPU."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("env", [{"DG_FORCE_TILE": "512"}, {"DG_FORCE_TILE": "3256"},
                                 {"DG_FORCE_TILE": "8256"},
                                 {"DG_FORCE_TILE": "4128"}, {"DG_FORCE_TILE": "264"},
                                 {"DG_TAIL_TILE": "8256"}, {"DG_TAIL_TILE": "4128"}, {"DG_TAIL_TILE": "264"},
                                 {"DG_FORCE_TILE": "256"}, {"DG_TAIL_TILE": "0"},
                                 {"DG_SPLITK": "1"}, {"DG_SPLITK": "3", "DG_FORCE_TILE": "4128"}],
                         ids=lambda e: "_".join(f"{k}={v}" for k, v in e.items()))
def test_tile_override(env):
    full = dict(os.environ)
    for k in ("DG_FORCE_TILE", "DG_TAIL_TILE", "DG_SPLITK"):
        full.pop(k, None)
    full.update(env)
    r = subprocess.run([sys.executable, os.path.join(HERE, "override_child.py")], env=full,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout, file=sys.stderr)
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]


def test_validate_offsets():
    """DG_VALIDATE=1: valid offsets give correct results, invalid ones are
    rejected on the host before any launch (tests/validate_child.py)."""
    full = dict(os.environ)
    full.pop("DG_FORCE_TILE", None)
    full.pop("DG_TAIL_TILE", None)
    full["DG_VALIDATE"] = "1"
    r = subprocess.run([sys.executable, os.path.join(HERE, "validate_child.py")], env=full,
                       capture_output=True, text=True, timeout=240)
    print(r.stdout, file=sys.stderr)
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
