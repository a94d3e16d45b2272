"""Seeded random shapes through the whole path against the fp64 oracle.

Each case draws widths (multiples of 8, not of 32), a set of adapters with
mixed ranks (0 and up to 128), random scales, token ids with -1 and unused
adapters, a token count from empty to large-batch size, and whether rows go
through token_rows, so that the planner picks every launch layout by itself
(small, medium and large batches, one or several launches). The fused
forward (y, u) and the packed backward (dx, dA, dB) are checked to the
parity bar.
"""
import numpy as np
import pytest

from helpers import BF16_TOL, FP32_TOL, GpuProblem, oracle_batch, rel_err, to_f64
from workloads import make_custom

pytestmark = pytest.mark.gpu

# (T, h_in, h_out, number of adapters); sizes kept so that the oracle finishes in seconds
SHAPES = [(0, 64, 40, 3), (1, 8, 8, 1), (37, 200, 264, 5), (300, 1032, 520, 12), (900, 264, 3080, 7),
          (2500, 520, 1032, 20), (4000, 2056, 264, 9), (17000, 264, 200, 6), (600, 4104, 72, 40),
          (1500, 72, 4104, 3)]


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_random_shapes_forward_backward(case):
    import torch
    import lora_adapter_batching_amd as L
    T, h_in, h_out, N = SHAPES[case]
    rng = np.random.default_rng(900 + case)
    ranks = [int(r) for r in rng.choice([0, 1, 4, 8, 12, 16, 24, 32, 40, 64, 96, 128], size=N)]
    if max(ranks) == 0:
        ranks[0] = 8
    ids = rng.integers(-1, N, size=T).astype(np.int32)
    if N > 2:
        ids[ids == N - 1] = 0  # one adapter without tokens
    prob = make_custom(950 + case, h_in, h_out, ranks, scales="random", ids=ids, with_dy=True, y0=bool(case % 2))
    gp = GpuProblem(prob, use_token_rows=bool(case % 3 == 1))
    ob = oracle_batch(prob)
    print(f"[case] fuzz {case}: T={T} {h_in}->{h_out} N={N} ranks={ranks} rows={gp.use_token_rows}", flush=True)
    y = gp.new_y()
    u = gp.new_u()
    ws = L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)
    L.sgmv_fused(gp.x, gp.adapters, gp.segments, y, u, ws)
    torch.cuda.synchronize()
    y_ref, u_ref = ob.forward()
    if T:
        assert rel_err(gp.sorted_rows(y), y_ref) <= BF16_TOL
        a = ob.token_adapter()
        ug = to_f64(u)
        for i in np.unique(a):
            if i >= 0 and ranks[i] > 0:
                m = a == i
                assert rel_err(ug[m, :ranks[i]], u_ref[m, :ranks[i]]) <= FP32_TOL, f"u adapter {i}"
    # backward from the forward's u, into NaN-filled gradients (all must be overwritten)
    dA = [torch.full((r, h_in), float("nan"), dtype=torch.float32, device="cuda") for r in ranks]
    dB = [torch.full((h_out, r), float("nan"), dtype=torch.float32, device="cuda") for r in ranks]
    pa = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dA], dtype=torch.int64, device="cuda")
    pb = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dB], dtype=torch.int64, device="cuda")
    dx = torch.zeros((T, h_in), dtype=torch.bfloat16, device="cuda")
    wsb = L.new_workspace(L.OP_BACKWARD, gp.adapters, gp.segments)
    L.packed_backward(gp.x, gp.dy, u, gp.adapters, gp.segments, dx, pa, pb, 0, wsb)
    torch.cuda.synchronize()
    du_ref, dx_ref, dA_ref, dB_ref = ob.backward()
    if T:
        assert rel_err(gp.sorted_rows(dx), dx_ref) <= BF16_TOL
    for i in range(N):
        if ranks[i] == 0:
            continue
        ga, gb = to_f64(dA[i]), to_f64(dB[i])
        assert not np.isnan(ga).any() and not np.isnan(gb).any(), f"adapter {i}: gradient not written"
        assert rel_err(ga, dA_ref[i]) <= FP32_TOL, f"dA[{i}]"
        assert rel_err(gb, dB_ref[i]) <= FP32_TOL, f"dB[{i}]"
