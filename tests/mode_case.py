"""One forward parity case under a forced launch layout (run as a child
process by test_gpu_modes.py: the layout override is read once per process).

Usage: LORA_SGMV_FORCE=<tile:NC | dep:KS:NC[:TICKS] | loc:KS:NC[:TICKS]> python mode_case.py <seed>
Prints one line "max_y_err max_u_err" and exits 0.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

from helpers import GpuProblem, oracle_batch, rel_err, to_f64  # noqa: E402
from workloads import make_custom  # noqa: E402


def main():
    import torch
    import lora_adapter_batching_amd as L
    seed = int(sys.argv[1])
    rng = np.random.default_rng(500 + seed)
    ranks = [8, 24, 12, 0, 128, 64, 16, 40, 1]
    ids = rng.integers(-1, len(ranks), size=700).astype(np.int32)
    prob = make_custom(seed, 1032, 360, ranks, scales="random", ids=ids, y0=True)
    gp = GpuProblem(prob, use_token_rows=bool(seed % 2))
    ob = oracle_batch(prob)
    L.load()
    y = gp.new_y()
    u = gp.new_u()
    ws = L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)
    for _ in range(2):  # the second call checks that counters returned to zero
        y.copy_(gp.y_init)
        L.sgmv_fused(gp.x, gp.adapters, gp.segments, y, u, ws)
    torch.cuda.synchronize()
    y_ref, u_ref = ob.forward()
    ey = rel_err(gp.sorted_rows(y), y_ref)
    a = ob.token_adapter()
    ug = to_f64(u)
    eu = 0.0
    for i in np.unique(a):
        if i < 0 or prob.ranks[i] == 0:
            continue
        m = a == i
        r = int(prob.ranks[i])
        eu = max(eu, rel_err(ug[m, :r], u_ref[m, :r]))
    print(f"{ey:.6e} {eu:.6e}", flush=True)


if __name__ == "__main__":
    main()
