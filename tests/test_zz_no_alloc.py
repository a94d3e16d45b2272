"""lora_sgmv_fused_noalloc (the fused call with the library's static device
scratch instead of a caller workspace) against lora_sgmv_fused with a
workspace, through the C ABI: two calls in a row on the same GPU, the
second with a smaller batch, each bit-identical to the workspace call and
within the parity tolerance of the fp64 oracle."""
import sys

import numpy as np
import pytest

from helpers import BF16_TOL, FP32_TOL, GpuProblem, oracle_batch, rel_err, to_f64
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def _compare(gp, label):
    import torch
    import lora_adapter_batching_amd as L
    ob = oracle_batch(gp.prob)
    y_ws, u_ws = gp.new_y(), gp.new_u()
    ws = L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)
    _say(f"{label}: lora_sgmv_fused with a workspace")
    L.sgmv_fused(gp.x, gp.adapters, gp.segments, y_ws, u_ws, ws)
    torch.cuda.synchronize()
    y_na, u_na = gp.new_y(), gp.new_u()
    _say(f"{label}: lora_sgmv_fused_noalloc")
    L.sgmv_fused_noalloc(gp.x, gp.adapters, gp.segments, y_na, u_na)
    torch.cuda.synchronize()
    # same kernels, same plan, deterministic sums: identical bits
    assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), f"{label}: y differs"
    assert torch.equal(torch.nan_to_num(u_na, nan=-7.0), torch.nan_to_num(u_ws, nan=-7.0)), f"{label}: u differs"
    y_ref, u_ref = ob.forward()
    e = rel_err(gp.sorted_rows(y_na), y_ref)
    assert e <= BF16_TOL, f"{label}: y rel err {e:.3e}"
    ug = to_f64(u_na)
    a = ob.token_adapter()
    for i in np.unique(a):
        if i < 0 or gp.prob.ranks[i] == 0:
            continue
        m = a == i
        r = int(gp.prob.ranks[i])
        assert rel_err(ug[m, :r], u_ref[m, :r]) <= FP32_TOL


def test_noalloc_matches_workspace_call_twice_second_smaller():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import lora_adapter_batching_amd as L
    L.load()
    # first call: the decode q projection (256 tokens, 8 adapters of rank 32,
    # split hand-off layout); second: a smaller request-order batch on the
    # same scratch (64 tokens, mixed ranks, an id -1 token, token_rows)
    big = make_config("decode")["q"]
    _compare(GpuProblem(big), "decode q 256 tok")
    rng = np.random.default_rng(3)
    ids = rng.integers(-1, 5, size=64).astype(np.int32)
    small = make_custom(21, 2560, 1024, [32, 16, 0, 64, 8], ids=ids, y0=True)
    _compare(GpuProblem(small, use_token_rows=True), "64 tok mixed ranks")
