"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
the same seeded inputs, element by element: at oracle-friendly sizes and at
the full workload sizes (every row of y / u / dx and every adapter's dA, dB).
"""
import copy
import sys

import numpy as np
import pytest

from oracle import oracle
from helpers import BF16_TOL, FP32_TOL, GpuProblem, dev_bf16, oracle_batch, rel_err, to_f64
from workloads import make_config, make_custom

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import lora_adapter_batching_amd as L
    L.load()
    yield


def _L():
    import lora_adapter_batching_amd as L
    return L


def _run_fused(gp, u=True, ws=None):
    L = _L()
    import torch
    y = gp.new_y()
    uu = gp.new_u() if u else None
    if ws is None:
        ws = L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)
    L.sgmv_fused(gp.x, gp.adapters, gp.segments, y, uu, ws)
    torch.cuda.synchronize()
    return y, uu


def _check_forward(gp, ob, y, u=None, rows=None):
    """Compare y (and u) at sorted positions `rows` (all if None)."""
    if rows is None:
        y_ref, u_ref = ob.forward()
        rows = np.arange(gp.prob.T)
    else:
        y_ref, u_ref = ob.forward_tokens(rows)
    yg = gp.sorted_rows(y)[rows]
    err = rel_err(yg, y_ref)
    assert err <= BF16_TOL, f"y rel err {err:.3e}"
    if u is not None:
        ug = to_f64(u)[rows]
        a = ob.token_adapter()[rows]
        for i in np.unique(a):
            if i < 0 or gp.prob.ranks[i] == 0:
                continue
            m = a == i
            r = int(gp.prob.ranks[i])
            e = rel_err(ug[m, :r], u_ref[m, :r])
            assert e <= FP32_TOL, f"u rel err {e:.3e} (adapter {i})"
    return err


# ---------------------------------------------------------------------------
# Tiny workload (16 decode tokens, 4 adapters of rank 8)
# ---------------------------------------------------------------------------
def test_tiny_fused_shrink_expand():
    L = _L()
    import torch
    prob = make_config("tiny")
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    assert np.array_equal(gp.perm, ob.perm)
    _say("tiny fused")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)
    _say("tiny shrink + expand")
    u2 = gp.new_u()
    ws = L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments)
    L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u2, ws)
    y2 = gp.new_y()
    L.sgmv_expand(u2, gp.adapters, gp.segments, y2)
    torch.cuda.synchronize()
    _check_forward(gp, ob, y2, u2)


# ---------------------------------------------------------------------------
# Mixed ranks, ragged shapes, -1 ids, empty segments, token_rows
# ---------------------------------------------------------------------------
def _mixed_problem(seed, T=300, h_in=264, h_out=200, y0=True):
    rng = np.random.default_rng(100 + seed)
    ranks = [8, 24, 12, 0, 128, 64, 16, 40, 1]
    ids = rng.integers(-1, len(ranks), size=T).astype(np.int32)
    ids[ids == 7] = 5  # adapter 7 gets no tokens (empty segment)
    return make_custom(seed, h_in, h_out, ranks, scales="random", ids=ids, y0=y0)


def test_weight_addresses_from_device_tables_and_host_copies():
    """Small launches take weight addresses from the host copies of the
    pointer tables when the caller gives them, else from the device tables:
    both against the oracle, and bit-identical to each other (fused, shrink
    and expand)."""
    L = _L()
    import torch
    prob = _mixed_problem(4)
    ob = oracle_batch(prob)
    outs = []
    for host_tables in (True, False):
        gp = GpuProblem(prob, host_tables=host_tables)
        assert len(gp.seg_adapter) <= 16
        _say(f"weight addresses host_tables={host_tables}")
        y, u = _run_fused(gp)
        _check_forward(gp, ob, y, u)
        u2 = gp.new_u()
        L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u2, L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments))
        y2 = gp.new_y()
        L.sgmv_expand(u2, gp.adapters, gp.segments, y2)
        torch.cuda.synchronize()
        _check_forward(gp, ob, y2, u2)
        outs.append([t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
                     for t in (y, u, y2, u2)])
    for a, b in zip(*outs):  # u starts as NaN: unwritten entries stay NaN in both
        assert np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("n_adapters", [16, 17])
@pytest.mark.parametrize("host_tables", [True, False])
def test_small_plan_capacity_edge(n_adapters, host_tables):
    """A batch of exactly as many segments as the small plan holds (16) and
    one more (17, the large plan): every segment a different rank, scale
    and weight address, so that each entry of the plan's tables (including
    the byte entries packed four to a word) is read for its own segment.
    Fused, shrink and expand against the oracle."""
    L = _L()
    import torch
    ranks = [1, 8, 12, 16, 24, 32, 40, 64, 96, 128, 4, 20, 48, 72, 100, 2, 56][:n_adapters]
    rng = np.random.default_rng(1600 + n_adapters)
    ids = np.concatenate([np.arange(n_adapters), rng.integers(0, n_adapters, size=80)]).astype(np.int32)
    rng.shuffle(ids)
    prob = make_custom(160 + n_adapters, 520, 264, ranks, scales="random", ids=ids, y0=True)
    gp = GpuProblem(prob, host_tables=host_tables)
    lens = np.diff(np.asarray(gp.seg_starts))
    active = [a for a, n in zip(gp.seg_adapter, lens) if a >= 0 and n > 0]
    assert len(active) == n_adapters  # segments with tokens and an adapter
    ob = oracle_batch(prob)
    _say(f"small-plan edge: {n_adapters} segments, host_tables={host_tables}")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)
    u2 = gp.new_u()
    L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u2, L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments))
    y2 = gp.new_y()
    L.sgmv_expand(u2, gp.adapters, gp.segments, y2)
    torch.cuda.synchronize()
    _check_forward(gp, ob, y2, u2)


@pytest.mark.parametrize("host_tables", [True, False])
def test_in_place_weight_update_and_table_swap(host_tables):
    """Adapters stay registered while their weights change: (1) new values
    written into the same A/B buffers between two calls (an optimizer step in
    place) and (2) the pointer table entries of two adapters re-pointed to a
    second set of buffers (double-buffered weights) are both picked up by the
    next call, each checked against the oracle on the new weights."""
    import torch
    L = _L()
    prob = _mixed_problem(6)
    gp = GpuProblem(prob, host_tables=host_tables)
    ws = L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)
    _say(f"in-place weight update host_tables={host_tables}")
    y, u = _run_fused(gp, ws=ws)
    _check_forward(gp, ob=oracle_batch(prob), y=y, u=u)
    # (1) in place: the same buffers, weights of another seed
    prob2 = make_custom(prob.seed + 100, prob.h_in, prob.h_out, list(prob.ranks), ids=prob.token_ids)
    for i in range(prob.N):
        if gp.A[i] is not None:
            gp.A[i].copy_(dev_bf16(prob2.A[i]))
            gp.B[i].copy_(dev_bf16(prob2.B[i]))
    upd = copy.copy(prob)  # same x, y0, ids and scales; the new weights
    upd.A, upd.B = list(prob2.A), list(prob2.B)
    y, u = _run_fused(gp, ws=ws)
    _check_forward(gp, ob=oracle_batch(upd), y=y, u=u)
    # (2) re-point adapters 0 and 4 to fresh buffers (device table, and the
    # host copies when the call carries them)
    prob3 = make_custom(prob.seed + 200, prob.h_in, prob.h_out, list(prob.ranks), ids=prob.token_ids)
    keep = []
    for i in (0, 4):
        a, b = dev_bf16(prob3.A[i]), dev_bf16(prob3.B[i])
        keep += [a, b]
        gp.adapters.A_ptrs[i] = a.data_ptr()
        gp.adapters.B_ptrs[i] = b.data_ptr()
        gp.adapters.A_host[i] = a.data_ptr()
        gp.adapters.B_host[i] = b.data_ptr()
        upd.A[i], upd.B[i] = prob3.A[i], prob3.B[i]
    y, u = _run_fused(gp, ws=ws)
    _check_forward(gp, ob=oracle_batch(upd), y=y, u=u)


@pytest.mark.parametrize("use_token_rows", [False, True])
def test_mixed_ranks_ragged(use_token_rows):
    L = _L()
    import torch
    prob = _mixed_problem(1)
    gp = GpuProblem(prob, use_token_rows=use_token_rows)
    ob = oracle_batch(prob)
    assert np.array_equal(gp.perm, ob.perm)
    _say(f"mixed fused token_rows={use_token_rows}")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)
    _say(f"mixed shrink/expand token_rows={use_token_rows}")
    u2 = gp.new_u()
    L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u2, L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments))
    y2 = gp.new_y()
    L.sgmv_expand(u2, gp.adapters, gp.segments, y2)
    torch.cuda.synchronize()
    _check_forward(gp, ob, y2, u2)
    # rows of tokens without a LoRA contribution are untouched (bitwise)
    a = ob.token_adapter()
    skip = np.array([i < 0 or prob.ranks[i] == 0 for i in a])
    y0 = gp.sorted_rows(gp.y_init)
    assert np.array_equal(gp.sorted_rows(y)[skip], y0[skip])


def test_fused_tile_mode_many_tokens():
    """Enough tiles that the planner picks the on-chip (fused-tile) mode."""
    prob = make_custom(7, 520, 392, [16, 32, 8, 72], scales="random",
                       seg_lens=[1500, 7, 1333, 33, 800, 700, 1], seg_adapter=[0, 1, 2, 3, 1, 0, 3])
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    _say("fused-tile mode, 4374 tokens")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)


def test_many_segments_split_launches():
    """More active segments than one launch plan holds."""
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 9, size=300).astype(np.int32)
    ad = rng.integers(-1, 6, size=300).astype(np.int32)
    prob = make_custom(8, 128, 96, [8, 16, 32, 4, 0, 48], scales="random", seg_lens=lens, seg_adapter=ad)
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    _say("300 segments fused")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)


def test_determinism_and_workspace_reuse():
    L = _L()
    import torch
    prob = _mixed_problem(2, y0=False)
    gp = GpuProblem(prob)
    ws = L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)
    _say("fused x3 same workspace")
    outs = []
    for _ in range(3):
        y, _ = _run_fused(gp, ws=ws)
        outs.append(to_f64(y))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])
    assert int(ws[:4096].to(torch.int32).abs().sum().item()) == 0, "counters not returned to zero"


def test_noop_cases():
    L = _L()
    import torch
    # rank-0 and zero-B adapters leave y unchanged
    prob = make_custom(9, 64, 48, [0, 8], ids=np.array([0, 1, 1, 0, 1], np.int32), y0=True)
    prob.B[1][:] = 0
    gp = GpuProblem(prob)
    _say("noop fused")
    y, _ = _run_fused(gp)
    assert np.array_equal(to_f64(y), to_f64(gp.y_init))
    # empty batch
    seg = L.Segments(np.array([0], np.int32), np.zeros(0, np.int32))
    y0 = torch.zeros((0, 48), dtype=torch.bfloat16, device="cuda")
    L.sgmv_fused(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), gp.adapters, seg, y0,
                 None, L.new_workspace(L.OP_FUSED, gp.adapters, seg))
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------
def test_decode_qwen3_4b_projections_full():
    projs = make_config("decode")
    for name, prob in projs.items():
        gp = GpuProblem(prob)
        ob = oracle_batch(prob)
        assert np.array_equal(gp.perm, ob.perm)
        _say(f"decode {name} {prob.h_in}->{prob.h_out}")
        y, u = _run_fused(gp)
        _check_forward(gp, ob, y, u)


@pytest.mark.parametrize("use_rows", [False, True])
def test_decode_shrink_then_expand_split_k(use_rows):
    """The separate shrink and expand calls on the decode projections: a
    decode batch has few tiles, so the shrink splits h_in = 2560 into parts
    whose last arriving workgroup sums them in order (per-tile counters that
    must return to zero: the call is made twice on one workspace)."""
    import torch
    L = _L()
    projs = make_config("decode")
    for name in ("q", "gate_up"):
        prob = projs[name]
        gp = GpuProblem(prob, use_token_rows=use_rows)
        ob = oracle_batch(prob)
        u = gp.new_u()
        ws = L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments)
        _say(f"decode {name} shrink (split k) + expand token_rows={use_rows}")
        for _ in range(2):
            y = gp.new_y()
            L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u, ws)
            L.sgmv_expand(u, gp.adapters, gp.segments, y, None)
        torch.cuda.synchronize()
        _check_forward(gp, ob, y, u)


def test_concurrent_calls_on_two_streams():
    """Two decode-sized fused calls (split hand-off layout) and a backward
    enqueued on two non-default streams at once, each with its own
    workspace: every result matches the oracle (hand-off state lives in the
    workspace and every launch has its own id)."""
    import torch
    L = _L()
    projs = make_config("decode")
    cases = []
    for name in ("q", "o"):
        prob = projs[name]
        gp = GpuProblem(prob)
        cases.append((gp, oracle_batch(prob), L.new_workspace(L.OP_FUSED, gp.adapters, gp.segments)))
    bprob = make_custom(51, 512, 384, [16, 64], seg_lens=[900, 700], seg_adapter=[0, 1], with_dy=True)
    bgp = GpuProblem(bprob)
    bws = L.new_workspace(L.OP_BACKWARD, bgp.adapters, bgp.segments)
    dA, dB, pa, pb = _grad_tables(bprob)
    dx = torch.zeros((bprob.T, bprob.h_in), dtype=torch.bfloat16, device="cuda")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    _say("concurrent fused calls and a backward on two streams")
    ys = [(k, cases[k][0].new_y()) for rep in range(3) for k in range(2)]
    torch.cuda.synchronize()
    # everything enqueued without a synchronisation in between: calls on one
    # stream share its workspace in order, the two streams run side by side
    for i, (k, y) in enumerate(ys):
        gp, _, ws = cases[k]
        L.sgmv_fused(gp.x, gp.adapters, gp.segments, y, None, ws, stream=streams[k])
        if i == 1:
            L.packed_backward(bgp.x, bgp.dy, None, bgp.adapters, bgp.segments, dx, pa, pb, 0, bws,
                              stream=streams[1])
    torch.cuda.synchronize()
    for k, y in ys:
        gp, ob, _ = cases[k]
        _check_forward(gp, ob, y)
    _check_backward(bgp, oracle_batch(bprob), dx, dA, dB)


def test_decode_request_order_token_rows_full():
    """Decode projections at full size with x and y left in request order:
    the kernels gather x rows and scatter y rows through token_rows."""
    projs = make_config("decode")
    for name, prob in projs.items():
        gp = GpuProblem(prob, use_token_rows=True)
        ob = oracle_batch(prob)
        _say(f"decode request order {name} {prob.h_in}->{prob.h_out}")
        y, u = _run_fused(gp)
        _check_forward(gp, ob, y, u)


def test_decode_request_order_host_row_copy():
    """Decode projections in request order with the row table passed only as
    a host copy (carried in the launch arguments, no device table): the
    oracle's result, and the same bits as the device-table call."""
    import torch
    projs = make_config("decode")
    for name, prob in projs.items():
        ob = oracle_batch(prob)
        outs = []
        for mode in ("only", ""):
            gp = GpuProblem(prob, use_token_rows=True, host_rows=mode)
            assert (gp.token_rows is None) == (mode == "only")
            _say(f"decode request order {name}, host rows {mode or 'none'}")
            y, u = _run_fused(gp)
            _check_forward(gp, ob, y, u)
            outs.append((y.view(torch.int16).cpu().numpy(), u.cpu().numpy()))
        assert np.array_equal(outs[0][0], outs[1][0])
        assert np.array_equal(outs[0][1], outs[1][1], equal_nan=True)


@pytest.mark.parametrize("mode", ["only", "both"])
def test_host_row_copy_shrink_expand_mixed(mode):
    """Mixed ranks, -1 ids and an empty segment in request order, the row
    table as a host copy (alone, or beside the device table): fused, shrink
    and expand against the oracle; rows without an adapter untouched."""
    L = _L()
    import torch
    prob = _mixed_problem(7, T=200)
    gp = GpuProblem(prob, use_token_rows=True, host_rows=mode)
    ob = oracle_batch(prob)
    _say(f"host row copy ({mode}) fused")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)
    _say(f"host row copy ({mode}) shrink / expand")
    u2 = gp.new_u()
    L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u2, L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments))
    y2 = gp.new_y()
    L.sgmv_expand(u2, gp.adapters, gp.segments, y2)
    torch.cuda.synchronize()
    _check_forward(gp, ob, y2, u2)
    a = ob.token_adapter()
    skip = np.array([i < 0 or prob.ranks[i] == 0 for i in a])
    assert np.array_equal(gp.sorted_rows(y)[skip], gp.sorted_rows(gp.y_init)[skip])


def test_token_rows_far_row_is_absent_not_wrapped():
    """A token_rows entry whose byte offset lies past 4 GiB (row 3 + 2^21 of a
    19456-wide bf16 matrix: the offset is row 3's plus a multiple of 2^32)
    is treated as absent by the forward and by the weight-gradient loads: its
    x / dy rows read as zero and its y / dx row is never written, and no
    other row changes (a 32-bit offset would have wrapped onto row 3)."""
    import torch
    L = _L()
    T, h_in, h_out = 64, 1024, 19456
    rng = np.random.default_rng(9)
    ids = rng.integers(0, 3, size=T).astype(np.int32)
    prob = make_custom(12, h_in, h_out, [16, 8, 32], ids=ids, with_dy=True, y0=True)
    gp = GpuProblem(prob, use_token_rows=True, y0=True)
    far = 3 + (1 << 21)
    # the far row must lie past the gather window of EVERY matrix the calls
    # touch (x and dx: h_in wide, y and dy: h_out wide): a row inside the
    # window is a real row, and one past the end of a small matrix would be
    # an access outside its allocation
    span = 0x7FFFFFF0
    for width in (h_in, h_out):
        off = far * width * 2
        assert off > span - 2 * width and off >= 1 << 32
        assert off % (1 << 32) == 3 * width * 2  # a 32-bit offset would land on row 3
    p_far = int(np.nonzero(gp.perm != 3)[0][5])  # a sorted position whose row is not row 3
    r_lost = int(gp.perm[p_far])
    rows = gp.perm.copy()
    rows[p_far] = far
    gp.token_rows.copy_(torch.from_numpy(rows))
    _say("token_rows far row: fused forward")
    y, u = _run_fused(gp)
    # reference: the same batch with position p_far's x row zero (so its u is
    # zero), and its y row left as it was
    pz = copy.deepcopy(prob)
    pz.x = prob.x.copy()
    pz.x[r_lost] = 0
    ob = oracle_batch(pz)
    y_ref, u_ref = ob.forward()
    yg = to_f64(y)
    y_ref_rows = np.empty_like(y_ref)
    y_ref_rows[gp.perm] = y_ref
    y_ref_rows[r_lost] = oracle.widen(prob.y0[r_lost])
    assert np.array_equal(yg[r_lost], y_ref_rows[r_lost]), "the absent row was written"
    assert rel_err(yg, y_ref_rows) <= BF16_TOL
    ug = to_f64(u)
    a = ob.token_adapter()
    for i in range(prob.N):
        m = a == i
        assert rel_err(ug[m, :prob.ranks[i]], u_ref[m, :prob.ranks[i]]) <= FP32_TOL
    assert np.all(ug[p_far, :prob.ranks[a[p_far]]] == 0.0)
    _say("token_rows far row: backward")
    pz.dy = prob.dy.copy()
    pz.dy[r_lost] = 0
    ob = oracle_batch(pz)
    dx, dA, dB = _run_backward(gp, u=None)
    du_ref, dx_ref, dA_ref, dB_ref = ob.backward()
    dxg = to_f64(dx)
    assert np.all(dxg[r_lost] == 0.0), "the absent dx row was written"
    dx_rows = np.zeros_like(dxg)
    dx_rows[gp.perm] = dx_ref
    dx_rows[r_lost] = 0.0
    assert rel_err(dxg, dx_rows) <= BF16_TOL
    for i in range(prob.N):
        assert rel_err(to_f64(dA[i]), dA_ref[i]) <= FP32_TOL, f"dA[{i}]"
        assert rel_err(to_f64(dB[i]), dB_ref[i]) <= FP32_TOL, f"dB[{i}]"


def test_decode_changing_batches_one_workspace():
    """Consecutive decode steps whose adapter ids change from step to step,
    as in serving: each step groups its ids, uploads its row table into the
    same device buffer and launches with the same workspace. Every step must
    match the oracle on its own batch (no hand-off state of an earlier step
    may leak into a later one)."""
    import torch
    L = _L()
    ranks = [32] * 8
    base = make_custom(41, 2560, 2560, ranks, ids=np.zeros(256, np.int32))
    A = [dev_bf16(a) for a in base.A]
    B = [dev_bf16(b) for b in base.B]
    ad = L.Adapters(A, B, base.ranks, base.scales, base.h_in, base.h_out)
    rows = torch.zeros(256, dtype=torch.int32, device="cuda")
    ws = None
    for step in range(4):
        rng = np.random.default_rng(100 + step)
        ids = rng.integers(-1 if step == 3 else 0, 8, size=256).astype(np.int32)
        prob = make_custom(41, 2560, 2560, ranks, ids=ids)  # same weights (same seed and shapes), new ids
        x = dev_bf16(prob.x)
        perm, starts, adap = L.segments_from_ids(ids, 8)
        rows.copy_(torch.from_numpy(perm))
        sg = L.Segments(starts, adap, rows)
        if ws is None:
            ws = L.new_workspace(L.OP_FUSED, ad, sg)
        y = torch.zeros((256, 2560), dtype=torch.bfloat16, device="cuda")
        _say(f"decode step {step} with changing ids")
        L.sgmv_fused(x, ad, sg, y, None, ws)
        torch.cuda.synchronize()
        y_ref, _ = oracle_batch(prob).forward()
        e = rel_err(to_f64(y)[perm], y_ref)
        assert e <= BF16_TOL, f"step {step}: y rel err {e:.3e}"


def test_prefill_llama3_8b_full():
    """Chunked prefill at full size: every row of y and u against the oracle."""
    prob = make_config("prefill")
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    _say("prefill 8192 tok 4096->4096")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)


def test_prefill_gather_shrink_expand_full():
    """Prefill at full size in request order (token_rows gather/scatter), and
    the separate shrink and expand entry points at full size; every row."""
    L = _L()
    import torch
    prob = make_config("prefill")
    gp = GpuProblem(prob, use_token_rows=True)
    ob = oracle_batch(prob)
    _say("prefill fused, token_rows")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)
    _say("prefill shrink + expand, token_rows")
    u2 = gp.new_u()
    L.sgmv_shrink(gp.x, gp.adapters, gp.segments, u2, L.new_workspace(L.OP_SHRINK, gp.adapters, gp.segments))
    y2 = gp.new_y()
    L.sgmv_expand(u2, gp.adapters, gp.segments, y2)
    torch.cuda.synchronize()
    _check_forward(gp, ob, y2, u2)


def test_hetero_mlp_up_full():
    """Heterogeneous ranks 8..128 with empty segments at full size: every
    row of y and u against the oracle."""
    prob = make_config("hetero")
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    assert np.array_equal(gp.perm, ob.perm)
    _say("hetero 4096 tok 4096->14336")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------
def _grad_tables(prob):
    import torch
    dA = [torch.full((int(r), prob.h_in), float("nan"), dtype=torch.float32, device="cuda")
          for r in prob.ranks]
    dB = [torch.full((prob.h_out, int(r)), float("nan"), dtype=torch.float32, device="cuda")
          for r in prob.ranks]
    pa = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dA], dtype=torch.int64, device="cuda")
    pb = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dB], dtype=torch.int64, device="cuda")
    return dA, dB, pa, pb


def _run_backward(gp, u=None, with_dx=True, flags=0, dA=None, dB=None):
    L = _L()
    import torch
    prob = gp.prob
    if dA is None:
        dA, dB, pa, pb = _grad_tables(prob)
    else:
        pa = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dA], dtype=torch.int64, device="cuda")
        pb = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dB], dtype=torch.int64, device="cuda")
    dx = torch.zeros((prob.T, prob.h_in), dtype=torch.bfloat16, device="cuda") if with_dx else None
    ws = L.new_workspace(L.OP_BACKWARD, gp.adapters, gp.segments)
    L.packed_backward(gp.x, gp.dy, u, gp.adapters, gp.segments, dx, pa, pb, flags, ws)
    torch.cuda.synchronize()
    return dx, dA, dB


def _check_backward(gp, ob, dx, dA, dB, adapters=None, dA0=None, dB0=None):
    prob = gp.prob
    if adapters is None:
        du_ref, dx_ref, dA_ref, dB_ref = ob.backward()
        rows = np.arange(prob.T)
        check = [i for i in range(prob.N) if prob.ranks[i] > 0]
    else:
        rows, du_ref, dx_ref, dA_ref, dB_ref = ob.backward_adapters(adapters)
        check = list(adapters)
    if dx is not None:
        e = rel_err(gp.sorted_rows(dx)[rows], dx_ref)
        assert e <= BF16_TOL, f"dx rel err {e:.3e}"
    for i in check:
        ga, gb = to_f64(dA[i]), to_f64(dB[i])
        ra = dA_ref[i] + (dA0[i] if dA0 is not None else 0.0)
        rb = dB_ref[i] + (dB0[i] if dB0 is not None else 0.0)
        ea, eb = rel_err(ga, ra), rel_err(gb, rb)
        assert ea <= FP32_TOL, f"dA[{i}] rel err {ea:.3e}"
        assert eb <= FP32_TOL, f"dB[{i}] rel err {eb:.3e}"


@pytest.mark.parametrize("mode", ["u_given", "u_recompute", "no_dx", "token_rows"])
def test_backward_mixed(mode):
    import torch
    rng = np.random.default_rng(3)
    ranks = [8, 24, 12, 0, 64, 16, 128, 40]
    T = 260
    ids = rng.integers(-1, len(ranks), size=T).astype(np.int32)
    ids[ids == 7] = 2  # adapter 7 has no tokens: its gradients must be zero
    prob = make_custom(11, 136, 200, ranks, scales="random", ids=ids, with_dy=True)
    gp = GpuProblem(prob, use_token_rows=(mode == "token_rows"))
    ob = oracle_batch(prob)
    u = None
    if mode != "u_recompute":
        _say(f"backward {mode}: forward for u")
        _, u = _run_fused(gp)
    _say(f"backward {mode}")
    dx, dA, dB = _run_backward(gp, u=u, with_dx=(mode != "no_dx"))
    _check_backward(gp, ob, dx, dA, dB)
    assert float(dA[7].abs().max()) == 0.0 and float(dB[7].abs().max()) == 0.0


@pytest.mark.parametrize("flags", [0, 1])
def test_backward_many_adapters_and_segments(flags):
    """70 adapters (two transpose groups, two weight-gradient launches) and
    one adapter spread over 150 segments (its token reduction is split into
    parts that must run in order)."""
    import torch
    L = _L()
    rng = np.random.default_rng(21)
    N = 70
    ranks = [int(r) for r in rng.choice([0, 4, 8, 16], size=N)]
    ranks[0] = 8
    lens, ads = [], []
    for g in range(150):  # adapter 0 in 150 short segments, interleaved with others
        lens.append(int(rng.integers(1, 4)))
        ads.append(0)
        lens.append(int(rng.integers(0, 5)))
        ads.append(int(rng.integers(-1, N)))
    prob = make_custom(22, 64, 40, ranks, scales="random", seg_lens=lens, seg_adapter=ads, with_dy=True)
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    dA0 = dB0 = None
    dA = dB = None
    if flags:
        g = np.random.default_rng(23)
        dA = [torch.tensor(g.standard_normal((r, prob.h_in)), dtype=torch.float32, device="cuda") for r in ranks]
        dB = [torch.tensor(g.standard_normal((prob.h_out, r)), dtype=torch.float32, device="cuda") for r in ranks]
        dA0 = [to_f64(t) for t in dA]
        dB0 = [to_f64(t) for t in dB]
    _say(f"backward 70 adapters, 300 segments, flags={flags}")
    dx, dA, dB = _run_backward(gp, u=None, flags=flags, dA=dA, dB=dB)
    _check_backward(gp, ob, dx, dA, dB, dA0=dA0, dB0=dB0)


def test_backward_accumulate():
    import torch
    rng = np.random.default_rng(4)
    ranks = [16, 32, 8]
    ids = rng.integers(0, 2, size=90).astype(np.int32)  # adapter 2 without tokens
    prob = make_custom(12, 96, 72, ranks, scales="random", ids=ids, with_dy=True)
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    dA0 = [np.random.default_rng(i).standard_normal((r, prob.h_in)) for i, r in enumerate(ranks)]
    dB0 = [np.random.default_rng(9 + i).standard_normal((prob.h_out, r)) for i, r in enumerate(ranks)]
    dA = [torch.tensor(a, dtype=torch.float32, device="cuda") for a in dA0]
    dB = [torch.tensor(b, dtype=torch.float32, device="cuda") for b in dB0]
    dA0 = [to_f64(t) for t in dA]
    dB0 = [to_f64(t) for t in dB]
    _say("backward accumulate")
    L = _L()
    dx, dA, dB = _run_backward(gp, u=None, flags=L.GRAD_ACCUMULATE, dA=dA, dB=dB)
    _check_backward(gp, ob, dx, dA, dB, dA0=dA0, dB0=dB0)
    assert np.array_equal(to_f64(dA[2]), dA0[2]) and np.array_equal(to_f64(dB[2]), dB0[2])


def test_train_qwen2p5_7b_full_size():
    """Packed training workload at full size: every row of y, u and dx, and
    dA_i / dB_i of all 32 adapters against the oracle (up to 32 adapters
    packed in one job: "Technische Samenvatting: PLoRA" (gist.science),
    "Belangrijkste Bijdragen")."""
    prob = make_config("train")
    gp = GpuProblem(prob)
    ob = oracle_batch(prob)
    _say("train forward 65536 tok 3584->3584")
    y, u = _run_fused(gp)
    _check_forward(gp, ob, y, u)
    del y
    _say("train backward")
    dx, dA, dB = _run_backward(gp, u=u)
    _check_backward(gp, ob, dx, dA, dB)


@pytest.mark.parametrize("flags,use_rows", [(0, False), (1, False), (0, True)])
def test_backward_split_token_ranges(flags, use_rows):
    """Few weight-gradient items for the GPU: the token ranges of the two
    heavy adapters are cut into parts that run side by side and are summed
    in a second pass (adapter 0 over three ragged segments, adapter 1 over
    one). A zero entry in the dB table skips that gradient (its buffer keeps
    its NaN fill) while its dA is still written."""
    import torch
    L = _L()
    ranks = [64, 8, 0, 32]
    lens = [700, 40, 900, 300, 63, 37]
    ads = [0, 2, 1, 0, 3, 0]
    prob = make_custom(31, 512, 384, ranks, scales="random", seg_lens=lens, seg_adapter=ads, with_dy=True)
    gp = GpuProblem(prob, use_token_rows=use_rows)
    ob = oracle_batch(prob)
    if flags:
        g = np.random.default_rng(32)
        dA = [torch.tensor(g.standard_normal((r, prob.h_in)), dtype=torch.float32, device="cuda") for r in ranks]
        dB = [torch.tensor(g.standard_normal((prob.h_out, r)), dtype=torch.float32, device="cuda") for r in ranks]
        dA0 = [to_f64(t) for t in dA]
        dB0 = [to_f64(t) for t in dB]
    else:
        dA, dB, _, _ = _grad_tables(prob)
        dA0 = dB0 = None
    pa = torch.tensor([t.data_ptr() if t.numel() else 0 for t in dA], dtype=torch.int64, device="cuda")
    pb = torch.tensor([t.data_ptr() if t.numel() and i != 1 else 0 for i, t in enumerate(dB)],
                      dtype=torch.int64, device="cuda")
    dB1_before = to_f64(dB[1]).copy()
    dx = torch.zeros((prob.T, prob.h_in), dtype=torch.bfloat16, device="cuda")
    ws = L.new_workspace(L.OP_BACKWARD, gp.adapters, gp.segments)
    _say(f"backward split token ranges flags={flags} token_rows={use_rows}")
    for _ in range(2):  # the second call reuses the workspace's partial slots
        if flags:
            for t, t0 in zip(dA, dA0):
                t.copy_(torch.from_numpy(t0).float())
            for t, t0 in zip(dB, dB0):
                t.copy_(torch.from_numpy(t0).float())
        dx.zero_()
        L.packed_backward(gp.x, gp.dy, None, gp.adapters, gp.segments, dx, pa, pb, flags, ws)
        torch.cuda.synchronize()
        du_ref, dx_ref, dA_ref, dB_ref = ob.backward()
        e = rel_err(gp.sorted_rows(dx), dx_ref)
        assert e <= BF16_TOL, f"dx rel err {e:.3e}"
        for i in (0, 1, 3):
            ra = dA_ref[i] + (dA0[i] if dA0 is not None else 0.0)
            ea = rel_err(to_f64(dA[i]), ra)
            assert ea <= FP32_TOL, f"dA[{i}] rel err {ea:.3e}"
            if i == 1:
                assert np.array_equal(np.isnan(to_f64(dB[1])), np.isnan(dB1_before))
                assert np.array_equal(np.nan_to_num(to_f64(dB[1]), nan=7.0), np.nan_to_num(dB1_before, nan=7.0))
                continue
            rb = dB_ref[i] + (dB0[i] if dB0 is not None else 0.0)
            eb = rel_err(to_f64(dB[i]), rb)
            assert eb <= FP32_TOL, f"dB[{i}] rel err {eb:.3e}"


def test_backward_split_is_deterministic():
    """Split weight gradients are bit-identical from call to call (the parts
    are added in a fixed order)."""
    import torch
    L = _L()
    ranks = [16]
    prob = make_custom(33, 256, 256, ranks, seg_lens=[3000], seg_adapter=[0], with_dy=True)
    gp = GpuProblem(prob)
    outs = []
    ws = L.new_workspace(L.OP_BACKWARD, gp.adapters, gp.segments)
    _say("backward split determinism")
    for _ in range(3):
        dA, dB, pa, pb = _grad_tables(prob)
        L.packed_backward(gp.x, gp.dy, None, gp.adapters, gp.segments, None, pa, pb, 0, ws)
        torch.cuda.synchronize()
        outs.append((to_f64(dA[0]), to_f64(dB[0])))
    for a, b in outs[1:]:
        assert np.array_equal(a, outs[0][0]) and np.array_equal(b, outs[0][1])
    ob = oracle_batch(prob)
    _, _, dA_ref, dB_ref = ob.backward()
    assert rel_err(outs[0][0], dA_ref[0]) <= FP32_TOL and rel_err(outs[0][1], dB_ref[0]) <= FP32_TOL


# ---------------------------------------------------------------------------
# Several projections over one x in one launch
# ---------------------------------------------------------------------------
MULTI_CASES = [
    # (T, h_in, outputs, adapters, rank choices, token_rows (True / "host"), host_tables)
    (256, 2560, (4096, 1024, 1024), 8, (32,), False, True),      # q/k/v-like decode, plan in device tables
    (256, 2560, (4096, 1024, 1024), 4, (8, 16, 32), True, True),  # small plan: weight addresses in the launch
    (100, 264, (72, 520), 3, (0, 1, 12, 40, 64), False, False),   # ragged widths, rank 0 in some projections
    (3000, 1032, (1032, 200, 3080, 8), 6, (8, 16, 24, 128), True, True),  # medium batch, four projections
    (18000, 264, (200, 264), 5, (8, 16, 32), False, True),        # large batch (one on-chip item per tile)
    # four projections of four adapters: 16 segments, the small plan's
    # capacity, so projection 3 sits in the last entries of its tables
    (200, 520, (264, 72, 136, 200), 4, (8, 16, 32, 64), False, True),
    # request order with the row table as a host copy alone (carried in the launch)
    (200, 520, (264, 72, 136), 4, (8, 16, 32, 64), "host", True),
]


@pytest.mark.parametrize("case", range(len(MULTI_CASES)))
def test_fused_multi_projection(case):
    """lora_sgmv_fused_multi: every projection's y matches the oracle of that
    projection alone (same x and ids, its own adapters)."""
    import torch
    L = _L()
    T, h_in, outs, N, choices, use_rows, host_tables = MULTI_CASES[case]
    rng = np.random.default_rng(700 + case)
    ids = rng.integers(-1, N, size=T).astype(np.int32)
    probs = []
    for p, h_out in enumerate(outs):
        ranks = [int(r) for r in rng.choice(choices, size=N)]
        pr = make_custom(710 + 10 * case + p, h_in, h_out, ranks, scales="random", ids=ids, y0=(p % 2 == 1))
        if probs:
            pr = copy.copy(pr)
            pr.x = probs[0].x  # one x for every projection
        probs.append(pr)
    gps = [GpuProblem(pr, use_token_rows=bool(use_rows), host_tables=host_tables,
                      host_rows="only" if use_rows == "host" else "") for pr in probs]
    ys = [g.new_y() for g in gps]
    ads = [g.adapters for g in gps]
    ws = L.new_workspace_multi(ads, gps[0].segments)
    _say(f"multi-projection case {case}: T={T} {h_in}->{outs} N={N} rows={use_rows}")
    for _ in range(2):  # the second call reuses the workspace (y accumulates twice)
        L.sgmv_fused_multi(gps[0].x, ads, gps[0].segments, ys, ws)
    torch.cuda.synchronize()
    for p, (g, pr, y) in enumerate(zip(gps, probs, ys)):
        ob = oracle_batch(pr)
        y_ref, _ = ob.forward()
        # two calls: y = y0 + 2 * delta
        y0 = to_f64(g.y_init)
        y0 = y0[g.perm] if g.use_token_rows else y0
        ref = y0 + 2.0 * (y_ref - y0)
        got = g.sorted_rows(y)
        if T:
            e = rel_err(got, ref)
            assert e <= BF16_TOL, f"projection {p}: y rel err {e:.3e}"


def test_workspace_sized_once_serves_smaller_batches():
    """One fused and one backward workspace, sized for the largest batch,
    serve later batches with fewer tokens and segments and other shapes of
    work (the layouts of small and medium batches use split hand-offs whose
    state lives in the workspace)."""
    import torch
    L = _L()
    ranks = [8, 32, 16, 64, 0, 24]
    big_ids = np.random.default_rng(60).integers(-1, len(ranks), size=3000).astype(np.int32)
    big = make_custom(61, 1032, 520, ranks, scales="random", ids=big_ids, with_dy=True)
    gbig = GpuProblem(big)
    wsf = L.new_workspace(L.OP_FUSED, gbig.adapters, gbig.segments)
    wsb = L.new_workspace(L.OP_BACKWARD, gbig.adapters, gbig.segments)
    for k, T in enumerate((3000, 257, 1, 900)):
        ids = np.random.default_rng(62 + k).integers(-1, len(ranks), size=T).astype(np.int32)
        prob = make_custom(61, 1032, 520, ranks, scales="random", ids=ids, with_dy=True)
        gp = GpuProblem(prob, use_token_rows=bool(k % 2))
        ob = oracle_batch(prob)
        _say(f"shared workspaces, batch {k}: T={T}")
        y, u = _run_fused(gp, ws=wsf)
        _check_forward(gp, ob, y, u)
        dA, dB, pa, pb = _grad_tables(prob)
        dx = torch.zeros((T, prob.h_in), dtype=torch.bfloat16, device="cuda")
        L.packed_backward(gp.x, gp.dy, u, gp.adapters, gp.segments, dx, pa, pb, 0, wsb)
        torch.cuda.synchronize()
        _check_backward(gp, ob, dx, dA, dB)
