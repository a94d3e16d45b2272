"""Pins for the fp64 CPU oracle, independent of the oracle's own code.

Each check ties the oracle to something else: a hand-worked example, numpy's
stable argsort, a dense brute-force product, torch autograd on a dense
formulation, finite differences, adjoint identities, or invariants that the
per-token low-rank update must satisfy. A dropped term, a wrong sign, a
transposed operand or a wrong index in lora_oracle.c fails at least one.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle
from workloads import make_custom, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _random_case(seed, T=37, h_in=24, h_out=40, ranks=(3, 0, 5, 8, 1), p_none=0.1):
    rng = np.random.default_rng(1000 + seed)
    N = len(ranks)
    ids = rng.integers(0, N, size=T).astype(np.int32)
    ids[rng.random(T) < p_none] = -1
    x = rng.standard_normal((T, h_in))
    A = [rng.standard_normal((r, h_in)) for r in ranks]
    B = [rng.standard_normal((h_out, r)) for r in ranks]
    s = rng.uniform(0.25, 4.0, size=N)
    y0 = rng.standard_normal((T, h_out))
    dy = rng.standard_normal((T, h_out))
    return dict(ids=ids, x=x, A=A, B=B, ranks=np.array(ranks, np.int32), s=s, y0=y0, dy=dy,
                N=N, T=T, h_in=h_in, h_out=h_out)


def _run_forward_ids(c, x=None, y0=None, A=None, B=None, s=None):
    perm, st, ad = oracle.segments_from_ids(c["ids"], c["N"])
    x = c["x"] if x is None else x
    y0 = c["y0"] if y0 is None else y0
    y, u = oracle.forward(x[perm], c["A"] if A is None else A, c["B"] if B is None else B,
                          c["ranks"], c["s"] if s is None else s, st, ad, y0[perm], c["h_out"])
    # back to request order
    yo = np.empty_like(y)
    yo[perm] = y
    uo = np.empty_like(u)
    uo[perm] = u
    return yo, uo


# --------------------------------------------------------------------------
# Hand-worked example (tests/golden/hand_example.json)
# --------------------------------------------------------------------------
def test_hand_example_exact():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    ids = np.array(g["ids_request_order"], np.int32)
    perm, st, ad = oracle.segments_from_ids(ids, len(g["ranks"]))
    assert perm.tolist() == g["expected_perm"]
    assert st.tolist() == g["expected_seg_starts"]
    assert ad.tolist() == g["expected_seg_adapter"]
    x = np.array(g["x_request_order"], np.float64)[perm]
    A = [np.array(a, np.float64) for a in g["A"]]
    B = [np.array(b, np.float64) for b in g["B"]]
    y, u = oracle.forward(x, A, B, g["ranks"], g["scales"], st, ad, None, g["h_out"])
    assert np.array_equal(y, np.array(g["expected_y_sorted"], np.float64))
    eu = np.array([[np.nan if v is None else v for v in row] for row in g["expected_u_sorted"]])
    assert np.array_equal(np.isnan(u), np.isnan(eu))
    assert np.array_equal(u[~np.isnan(u)], eu[~np.isnan(eu)])
    dy = np.array(g["dy_sorted"], np.float64)
    du, dx, dA, dB = oracle.backward(x, dy, u, A, B, g["ranks"], g["scales"], st, ad)
    edu = np.array([[np.nan if v is None else v for v in row] for row in g["expected_du_sorted"]])
    assert np.array_equal(np.isnan(du), np.isnan(edu))
    assert np.array_equal(du[~np.isnan(du)], edu[~np.isnan(edu)])
    assert np.array_equal(dx, np.array(g["expected_dx_sorted"], np.float64))
    for i in range(2):
        assert np.array_equal(dA[i], np.array(g["expected_dA"][i], np.float64))
        assert np.array_equal(dB[i], np.array(g["expected_dB"][i], np.float64))


# --------------------------------------------------------------------------
# Bookkeeping: grouping ids into segments
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_segments_match_numpy_stable_argsort(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 40))
    T = int(rng.integers(0, 3000))
    ids = rng.integers(-1, N, size=T).astype(np.int32)
    perm, st, ad = oracle.segments_from_ids(ids, N)
    key = np.where(ids < 0, N, ids)
    assert np.array_equal(perm, np.argsort(key, kind="stable").astype(np.int32))
    counts = np.bincount(key, minlength=N + 1)
    assert np.array_equal(st, np.concatenate([[0], np.cumsum(counts)]).astype(np.int32))
    assert np.array_equal(ad, np.concatenate([np.arange(N), [-1]]).astype(np.int32))


def test_segments_reject_bad_ids():
    with pytest.raises(ValueError):
        oracle.segments_from_ids(np.array([0, 3], np.int32), 3)
    with pytest.raises(ValueError):
        oracle.segments_from_ids(np.array([-2], np.int32), 3)


# --------------------------------------------------------------------------
# Forward pins
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_forward_matches_dense_delta_w(seed):
    """Brute force: dense Delta W_i = s_i B_i A_i, then y = y0 + Delta W_i x
    per token (numpy matmul)."""
    c = _random_case(seed)
    y, u = _run_forward_ids(c)
    ref = c["y0"].copy()
    for t in range(c["T"]):
        i = c["ids"][t]
        if i < 0:
            continue
        dW = c["s"][i] * (c["B"][i] @ c["A"][i])
        ref[t] += dW @ c["x"][t]
    assert _rel(y, ref) < 1e-12
    for t in range(c["T"]):
        i = c["ids"][t]
        if i >= 0 and c["ranks"][i] > 0:
            assert _rel(u[t, :c["ranks"][i]], c["A"][i] @ c["x"][t]) < 1e-12


def test_forward_single_adapter_is_two_gemms():
    rng = np.random.default_rng(7)
    T, h_in, h_out, r = 19, 33, 21, 6
    x = rng.standard_normal((T, h_in))
    A = rng.standard_normal((r, h_in))
    B = rng.standard_normal((h_out, r))
    y0 = rng.standard_normal((T, h_out))
    y, u = oracle.forward(x, [A], [B], [r], [1.5], [0, T], [0], y0, h_out)
    assert _rel(u, x @ A.T) < 1e-13
    assert _rel(y, y0 + 1.5 * (x @ A.T) @ B.T) < 1e-13


def test_forward_noop_cases_leave_y_unchanged():
    """Rank 0, an all-zero B, id -1 and empty segments leave y unchanged (by value)."""
    rng = np.random.default_rng(3)
    T, h_in, h_out = 12, 16, 10
    x = rng.standard_normal((T, h_in))
    y0 = rng.standard_normal((T, h_out))
    A = [rng.standard_normal((0, h_in)), rng.standard_normal((4, h_in)),
         rng.standard_normal((5, h_in))]
    B = [np.zeros((h_out, 0)), np.zeros((h_out, 4)), rng.standard_normal((h_out, 5))]
    # segments: rank-0 adapter, zero-B adapter, no-adapter, empty segment of adapter 2
    st = np.array([0, 4, 8, 12, 12], np.int32)
    ad = np.array([0, 1, -1, 2], np.int32)
    y, _ = oracle.forward(x, A, B, [0, 4, 5], [2.0, 2.0, 2.0], st, ad, y0, h_out)
    assert np.array_equal(y, y0)


def test_forward_linear_in_x_and_scale():
    c = _random_case(11)
    z = np.zeros_like(c["y0"])
    x2 = np.random.default_rng(5).standard_normal(c["x"].shape)
    ya, _ = _run_forward_ids(c, y0=z)
    yb, _ = _run_forward_ids(c, x=x2, y0=z)
    yab, _ = _run_forward_ids(c, x=c["x"] + 2.0 * x2, y0=z)
    assert _rel(yab, ya + 2.0 * yb) < 1e-12
    y3, _ = _run_forward_ids(c, y0=z, s=3.0 * c["s"])
    assert _rel(y3, 3.0 * ya) < 1e-12


def test_forward_adapter_relabel_and_segment_split_and_permutation():
    c = _random_case(13)
    y, _ = _run_forward_ids(c)
    # relabel adapters with a permutation
    N = c["N"]
    q = np.random.default_rng(1).permutation(N)
    ids2 = np.where(c["ids"] < 0, -1, q[np.maximum(c["ids"], 0)]).astype(np.int32)
    inv = np.argsort(q)
    c2 = dict(c, ids=ids2, A=[c["A"][inv[j]] for j in range(N)],
              B=[c["B"][inv[j]] for j in range(N)], ranks=c["ranks"][inv], s=c["s"][inv])
    y2, _ = _run_forward_ids(c2)
    assert np.array_equal(y, y2)
    # split every segment in two (same adapter): identical result
    perm, st, ad = oracle.segments_from_ids(c["ids"], N)
    st2, ad2 = [0], []
    for g in range(len(ad)):
        mid = (st[g] + st[g + 1]) // 2
        st2 += [mid, st[g + 1]]
        ad2 += [ad[g], ad[g]]
    ys, _ = oracle.forward(c["x"][perm], c["A"], c["B"], c["ranks"], c["s"], st, ad,
                           c["y0"][perm], c["h_out"])
    ys2, _ = oracle.forward(c["x"][perm], c["A"], c["B"], c["ranks"], c["s"],
                            np.array(st2, np.int32), np.array(ad2, np.int32), c["y0"][perm],
                            c["h_out"])
    assert np.array_equal(ys, ys2)
    # permuting the request order changes nothing per token (bit-identical)
    p = np.random.default_rng(2).permutation(c["T"])
    c3 = dict(c, ids=c["ids"][p], x=c["x"][p], y0=c["y0"][p])
    y3, _ = _run_forward_ids(c3)
    assert np.array_equal(y3, y[p])


# --------------------------------------------------------------------------
# Backward pins
# --------------------------------------------------------------------------
def _torch_dense_reference(c, perm, st, ad):
    """Autograd of the dense formulation y = y0 + s_i (x A_i^T) B_i^T per
    segment; returns grads w.r.t. x (sorted order), A_i, B_i and u."""
    xs = torch.tensor(c["x"][perm], dtype=torch.float64, requires_grad=True)
    A = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in c["A"]]
    B = [torch.tensor(b, dtype=torch.float64, requires_grad=True) for b in c["B"]]
    dy = torch.tensor(c["dy"][perm], dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    us = []
    for g in range(len(ad)):
        i = int(ad[g])
        a, b = int(st[g]), int(st[g + 1])
        if i < 0 or c["ranks"][i] == 0 or a == b:
            continue
        u = xs[a:b] @ A[i].T
        u.retain_grad()
        us.append((a, b, i, u))
        y = c["s"][i] * (u @ B[i].T)
        loss = loss + (dy[a:b] * y).sum()
    loss.backward()
    zero = lambda t, shape: (t.grad.numpy() if t.grad is not None else np.zeros(shape))
    gx = xs.grad.numpy() if xs.grad is not None else np.zeros(xs.shape)
    gA = [zero(a, a.shape) for a in A]
    gB = [zero(b, b.shape) for b in B]
    gu = {(a, b): u.grad.numpy() for (a, b, i, u) in us}
    return gx, gA, gB, gu


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_torch_autograd(seed):
    c = _random_case(20 + seed)
    perm, st, ad = oracle.segments_from_ids(c["ids"], c["N"])
    xs, dys = c["x"][perm], c["dy"][perm]
    _, u = oracle.forward(xs, c["A"], c["B"], c["ranks"], c["s"], st, ad, None, c["h_out"])
    du, dx, dA, dB = oracle.backward(xs, dys, u, c["A"], c["B"], c["ranks"], c["s"], st, ad)
    gx, gA, gB, gu = _torch_dense_reference(c, perm, st, ad)
    assert _rel(dx, gx) < 1e-12
    for i in range(c["N"]):
        if c["ranks"][i]:
            assert _rel(dA[i], gA[i]) < 1e-12
            assert _rel(dB[i], gB[i]) < 1e-12
    for (a, b), g in gu.items():
        r = g.shape[1]
        assert _rel(du[a:b, :r], g) < 1e-12


def test_backward_finite_differences():
    """L = sum(dy * y) is linear in each of x, A_i, B_i on its own, so central
    differences are exact up to rounding."""
    c = _random_case(31, T=15, h_in=9, h_out=7, ranks=(2, 3, 0))
    perm, st, ad = oracle.segments_from_ids(c["ids"], c["N"])
    z = np.zeros((c["T"], c["h_out"]))

    def loss(x=None, A=None, B=None):
        y, _ = oracle.forward((c["x"] if x is None else x)[perm], c["A"] if A is None else A,
                              c["B"] if B is None else B, c["ranks"], c["s"], st, ad, z,
                              c["h_out"])
        return float(np.sum(c["dy"][perm] * y))

    xs = c["x"][perm]
    _, u = oracle.forward(xs, c["A"], c["B"], c["ranks"], c["s"], st, ad, None, c["h_out"])
    du, dx, dA, dB = oracle.backward(xs, c["dy"][perm], u, c["A"], c["B"], c["ranks"], c["s"],
                                     st, ad)
    h = 1e-3
    rng = np.random.default_rng(0)
    for _ in range(6):
        t, d = int(rng.integers(c["T"])), int(rng.integers(c["h_in"]))
        xp, xm = c["x"].copy(), c["x"].copy()
        xp[t, d] += h
        xm[t, d] -= h
        fd = (loss(x=xp) - loss(x=xm)) / (2 * h)
        p = int(np.nonzero(perm == t)[0][0])
        assert abs(fd - dx[p, d]) <= 1e-8 * max(1.0, abs(fd))
    for i in (0, 1):
        r = c["ranks"][i]
        for _ in range(4):
            k, d = int(rng.integers(r)), int(rng.integers(c["h_in"]))
            Ap = [a.copy() for a in c["A"]]
            Am = [a.copy() for a in c["A"]]
            Ap[i][k, d] += h
            Am[i][k, d] -= h
            fd = (loss(A=Ap) - loss(A=Am)) / (2 * h)
            assert abs(fd - dA[i][k, d]) <= 1e-8 * max(1.0, abs(fd))
            j, k2 = int(rng.integers(c["h_out"])), int(rng.integers(r))
            Bp = [b.copy() for b in c["B"]]
            Bm = [b.copy() for b in c["B"]]
            Bp[i][j, k2] += h
            Bm[i][j, k2] -= h
            fd = (loss(B=Bp) - loss(B=Bm)) / (2 * h)
            assert abs(fd - dB[i][j, k2]) <= 1e-8 * max(1.0, abs(fd))


def test_backward_adjoint_identities():
    """<dy, J_x v> = <dx, v>, <dy, J_A V> = sum <dA_i, V_i>, <dy, J_B W> = sum <dB_i, W_i>:
    y - y0 is linear in x, in A (fixed B) and in B (fixed A)."""
    c = _random_case(41)
    perm, st, ad = oracle.segments_from_ids(c["ids"], c["N"])
    xs, dys = c["x"][perm], c["dy"][perm]
    z = np.zeros((c["T"], c["h_out"]))
    _, u = oracle.forward(xs, c["A"], c["B"], c["ranks"], c["s"], st, ad, None, c["h_out"])
    du, dx, dA, dB = oracle.backward(xs, dys, u, c["A"], c["B"], c["ranks"], c["s"], st, ad)
    rng = np.random.default_rng(9)
    v = rng.standard_normal(xs.shape)
    yv, _ = oracle.forward(v, c["A"], c["B"], c["ranks"], c["s"], st, ad, z, c["h_out"])
    assert abs(np.sum(dys * yv) - np.sum(dx * v)) < 1e-10 * np.sum(np.abs(dys * yv))
    V = [rng.standard_normal(a.shape) for a in c["A"]]
    yV, _ = oracle.forward(xs, V, c["B"], c["ranks"], c["s"], st, ad, z, c["h_out"])
    lhs = np.sum(dys * yV)
    rhs = sum(np.sum(dA[i] * V[i]) for i in range(c["N"]))
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))
    W = [rng.standard_normal(b.shape) for b in c["B"]]
    yW, _ = oracle.forward(xs, c["A"], W, c["ranks"], c["s"], st, ad, z, c["h_out"])
    lhs = np.sum(dys * yW)
    rhs = sum(np.sum(dB[i] * W[i]) for i in range(c["N"]))
    assert abs(lhs - rhs) < 1e-10 * max(1.0, abs(lhs))


def test_backward_accumulate_and_unused_adapters():
    c = _random_case(51, ranks=(3, 4, 2))
    c["ids"][c["ids"] == 2] = 0  # adapter 2 has no tokens
    perm, st, ad = oracle.segments_from_ids(c["ids"], c["N"])
    xs, dys = c["x"][perm], c["dy"][perm]
    _, u = oracle.forward(xs, c["A"], c["B"], c["ranks"], c["s"], st, ad, None, c["h_out"])
    _, dx, dA, dB = oracle.backward(xs, dys, u, c["A"], c["B"], c["ranks"], c["s"], st, ad)
    assert not np.any(dA[2]) and not np.any(dB[2])
    dx0 = np.random.default_rng(2).standard_normal(dx.shape)
    dA0 = [np.full(a.shape, 1.25) for a in dA]
    dB0 = [np.full(b.shape, -0.5) for b in dB]
    _, dx2, dA2, dB2 = oracle.backward(xs, dys, u, c["A"], c["B"], c["ranks"], c["s"], st, ad,
                                       dx0=dx0, dA0=dA0, dB0=dB0, accumulate=True)
    assert _rel(dx2, dx + dx0) < 1e-14
    for i in range(3):
        assert _rel(dA2[i], dA[i] + 1.25) < 1e-14
        assert _rel(dB2[i], dB[i] - 0.5) < 1e-14


def test_backward_permutation_invariance_of_weight_grads():
    c = _random_case(61)
    perm, st, ad = oracle.segments_from_ids(c["ids"], c["N"])
    _, u = oracle.forward(c["x"][perm], c["A"], c["B"], c["ranks"], c["s"], st, ad, None,
                          c["h_out"])
    _, _, dA, dB = oracle.backward(c["x"][perm], c["dy"][perm], u, c["A"], c["B"], c["ranks"],
                                   c["s"], st, ad)
    p = np.random.default_rng(3).permutation(c["T"])
    c2 = dict(c, ids=c["ids"][p], x=c["x"][p], dy=c["dy"][p])
    perm2, st2, ad2 = oracle.segments_from_ids(c2["ids"], c2["N"])
    _, u2 = oracle.forward(c2["x"][perm2], c["A"], c["B"], c["ranks"], c["s"], st2, ad2, None,
                           c["h_out"])
    _, _, dA2, dB2 = oracle.backward(c2["x"][perm2], c2["dy"][perm2], u2, c["A"], c["B"],
                                     c["ranks"], c["s"], st2, ad2)
    for i in range(c["N"]):
        if c["ranks"][i]:
            assert _rel(dA2[i], dA[i]) < 1e-12 and _rel(dB2[i], dB[i]) < 1e-12


def test_thread_count_does_not_change_results():
    c = _random_case(71, T=64)
    n0 = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        y1, _ = _run_forward_ids(c)
        oracle.set_num_threads(max(2, n0))
        y2, _ = _run_forward_ids(c)
    finally:
        oracle.set_num_threads(n0)
    assert np.array_equal(y1, y2)


# --------------------------------------------------------------------------
# Workload generator sanity (shapes, grouping recipe) -- not method arithmetic
# --------------------------------------------------------------------------
def test_workload_tiny_shapes_and_bf16_rounding():
    p = make_config("tiny")
    assert p.T == 16 and p.h_in == 256 and p.h_out == 256 and p.N == 4
    assert all(a.shape == (8, 256) for a in p.A) and all(b.shape == (256, 8) for b in p.B)
    f = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    from workloads import bf16_bits_from_f32
    ours = bf16_bits_from_f32(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_workload_custom_is_deterministic():
    a = make_custom(5, 64, 48, [8, 16], ids=np.array([0, 1, 1, -1, 0], np.int32))
    b = make_custom(5, 64, 48, [8, 16], ids=np.array([0, 1, 1, -1, 0], np.int32))
    assert np.array_equal(a.x, b.x) and all(np.array_equal(p, q) for p, q in zip(a.A, b.A))


# --------------------------------------------------------------------------
# The Python helpers that feed the oracle: bf16 widening and the row /
# adapter restrictions that build the references of the large parity checks
# --------------------------------------------------------------------------
def test_widen_matches_torch_on_every_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # float32 -> float64 of signalling NaN patterns
        ours = oracle.widen(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    # 2 * (2^7 - 1) NaN payloads per sign: exponent all ones, mantissa non-zero
    assert int(nan.sum()) == 2 * 127
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # the sign bit survives on zeros, and the extremes are what IEEE fixes
    assert ours[0x0000] == 0.0 and not np.signbit(ours[0x0000])
    assert ours[0x8000] == 0.0 and np.signbit(ours[0x8000])
    assert ours[0x7F80] == np.inf and ours[0xFF80] == -np.inf
    assert ours[0x3F80] == 1.0 and ours[0xC000] == -2.0
    assert ours[0x0001] == 2.0 ** -133          # smallest subnormal
    assert ours[0x007F] == 127 * 2.0 ** -133    # largest subnormal
    assert ours[0x0080] == 2.0 ** -126          # smallest normal
    assert ours[0x7F7F] == (2 - 2.0 ** -7) * 2.0 ** 127  # largest finite
    # a 2-D array keeps its shape and row order
    m = bits[:12].reshape(3, 4)
    assert np.array_equal(oracle.widen(m), ours[:12].reshape(3, 4))


def _helper_problem():
    # request-order ids over 5 adapters (one of rank 0), with -1 tokens, an
    # upstream gradient and a non-zero initial y
    rng = np.random.default_rng(77)
    ids = rng.integers(-1, 5, size=53).astype(np.int32)
    return make_custom(11, 40, 24, [3, 8, 0, 5, 16], scales="random", ids=ids, with_dy=True, y0=True)


def _nan_equal(a, b):
    return np.array_equal(np.asarray(a), np.asarray(b), equal_nan=True)


def test_batch_forward_tokens_equals_rows_of_forward():
    p = _helper_problem()
    ob = oracle.Batch(p)
    y, u = ob.forward()
    rng = np.random.default_rng(3)
    for rows in (np.arange(p.T), rng.permutation(p.T)[:17], np.array([p.T - 1, 0, 5, 5])):
        yr, ur = ob.forward_tokens(rows)
        # each token is computed on its own in the same order: bit-identical
        assert _nan_equal(yr, y[rows])
        assert _nan_equal(ur, u[rows][:, :ur.shape[1]])
    # an id -1 token keeps its initial row and leaves u unwritten
    a = ob.token_adapter()
    r = np.nonzero(a < 0)[0]
    assert r.size > 0
    yr, ur = ob.forward_tokens(r)
    assert np.array_equal(yr, ob.y0[r]) and np.all(np.isnan(ur))


def test_batch_backward_adapters_equals_full_backward():
    p = _helper_problem()
    ob = oracle.Batch(p)
    du, dx, dA, dB = ob.backward()
    a = ob.token_adapter()
    for subset in ([0], [3, 1], [4, 0, 1, 3], [2]):
        rows, dus, dxs, dAs, dBs = ob.backward_adapters(subset)
        assert np.array_equal(rows, np.nonzero(np.isin(a, subset))[0])
        # the token sums run over the same tokens in the same ascending order
        for i in subset:
            assert np.array_equal(dAs[i], dA[i]) and np.array_equal(dBs[i], dB[i])
        # adapters outside the subset get no contribution
        for i in set(range(p.N)) - set(subset):
            assert not np.any(dAs[i]) and not np.any(dBs[i])
        assert _nan_equal(dus, du[rows][:, :dus.shape[1]])
        assert np.array_equal(dxs, dx[rows])
