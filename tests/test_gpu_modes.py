"""Every launch layout of the fused kernel against the fp64 oracle.

The planner picks one layout per call from the batch shape; these cases force
each layout (on-chip tile, split shrink with waiting expands, the same with
every item of a tile on one XCD, several k-chunk and column-chunk counts, and
expands that give up waiting at once and recompute the shrink) on one ragged
mixed-rank batch, in a child process because the override is read once per
process.
"""
import os
import subprocess
import sys

import pytest

from helpers import BF16_TOL, FP32_TOL

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("layout,seed", [("tile:1", 0), ("tile:5", 1), ("dep:1:3", 2), ("dep:3:4", 3),
                                         ("dep:9:2", 4), ("dep:3:4:0", 5), ("loc:1:3", 6), ("loc:4:5", 7),
                                         ("loc:9:2", 8), ("loc:4:5:0", 9)])
def test_forced_layout(layout, seed):
    print(f"[case] forced layout {layout} seed {seed}", flush=True)
    env = dict(os.environ, LORA_SGMV_FORCE=layout)
    r = subprocess.run([sys.executable, os.path.join(HERE, "mode_case.py"), str(seed)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    ey, eu = (float(v) for v in r.stdout.strip().splitlines()[-1].split())
    assert ey <= BF16_TOL, f"y rel err {ey:.3e} under {layout}"
    assert eu <= FP32_TOL, f"u rel err {eu:.3e} under {layout}"
