"""GPU checks of the device-planned decode call (lora_sgmv_fused_graph).

The pages' serving engine keeps decoding while updated adapter weights are
loaded in place ("Trajectory presenta C-LoRA" (vivodigitale.it), "Come
funziona l'architettura"). These tests capture the call into a HIP graph and
replay it with new ids, weights, scales, ranks and re-pointed tables, each
replay against the fp64 oracle; and they overwrite one adapter's second
weight buffer on another stream while a decode reads the first buffer.
"""
import sys

import numpy as np
import pytest

from helpers import BF16_TOL, dev_bf16, rel_err, to_f64
from oracle import oracle
from workloads import make_custom

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


class _Tables:
    """Device tables of a graph call plus the host copies the oracle uses."""

    def __init__(self, prob, max_rank):
        import torch
        import lora_adapter_batching_amd as L
        self.h_in, self.h_out = prob.h_in, prob.h_out
        self.A_bits = [a.copy() for a in prob.A]
        self.B_bits = [b.copy() for b in prob.B]
        self.ranks = np.array(prob.ranks, np.int32)
        self.scales = np.array(prob.scales, np.float32)
        self.A = [dev_bf16(a) if a.size else None for a in self.A_bits]
        self.B = [dev_bf16(b) if b.size else None for b in self.B_bits]
        self.A_ptrs = torch.tensor([t.data_ptr() if t is not None else 0 for t in self.A], dtype=torch.int64,
                                   device="cuda")
        self.B_ptrs = torch.tensor([t.data_ptr() if t is not None else 0 for t in self.B], dtype=torch.int64,
                                   device="cuda")
        self.ranks_dev = torch.from_numpy(self.ranks.copy()).cuda()
        self.scales_dev = torch.from_numpy(self.scales.copy()).cuda()
        self.ga = L.GraphAdapters(self.A_ptrs, self.B_ptrs, self.ranks_dev, self.scales_dev, prob.h_in,
                                  prob.h_out, max_rank)

    def oracle_y(self, x_bits, y0_bits, ids):
        """fp64 reference in request order (ids outside [0, N) or inactive
        adapters leave their row as it was)."""
        N = len(self.ranks)
        key = np.array([i if 0 <= i < N and self.ranks[i] > 0 else -1 for i in ids], np.int32)
        perm, st, ad = oracle.segments_from_ids(key, N)
        x = oracle.widen(x_bits)[perm]
        y0 = oracle.widen(y0_bits)[perm]
        A = [oracle.widen(a) for a in self.A_bits]
        B = [oracle.widen(b) for b in self.B_bits]
        y, _ = oracle.forward(x, A, B, self.ranks, self.scales.astype(np.float64), st, ad, y0, self.h_out)
        out = np.empty_like(y)
        out[perm] = y
        return out


def _problem(seed, T, h_in, h_out, ranks):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, len(ranks), size=T).astype(np.int32)
    return make_custom(seed, h_in, h_out, ranks, scales="random", ids=ids, y0=True)


CASES = [
    # decode-like q projection: 256 tokens, 8 adapters of rank 32 (XCD-local split layout)
    ("q_2560", 256, 2560, 2560, [32] * 8, 32),
    # expand-heavy MLP-up-like projection, mixed ranks (split layout over all XCDs)
    ("up_1024x8192", 64, 1024, 8192, [8, 16, 0, 64, 32], 64),
    # the most tokens a launch plans by itself; 13 adapters, one inactive
    ("q_1024tok_13ad", 1024, 2048, 1024, [16] * 12 + [0], 16),
    # more tokens than a launch plans by itself: the plan kernel runs first
    ("o_1500tok_plan_kernel", 1500, 1024, 2048, [32] * 8, 32),
    # ranks 8..128 (every rank-block count), some adapters without weights
    ("r8_128_40ad_700tok", 700, 1024, 1536, ([8, 16, 32, 64, 128, 0, 24, 40] * 5), 128),
    # the most adapters a device-planned call takes, rank 4 (V rows shorter
    # than 16 bytes), about two tokens each
    ("r4_256ad_512tok", 512, 512, 512, [4] * 256, 4),
    # a single token
    ("one_token", 1, 256, 512, [8, 8], 8),
    # the decode gate_up projection at full size (the graph-replay bench's widest call)
    ("gate_up_2560x19456", 256, 2560, 19456, [32] * 8, 32),
    # the widest count scan (256 adapters: keys in every lane of the wave),
    # planned inside the launch at its token limit and by the plan kernel
    ("scan_256ad_1024tok", 1024, 512, 264, [8, 16, 4, 32, 0, 24, 12, 40] * 32, 40),
    ("scan_256ad_2048tok", 2048, 264, 512, [16, 8, 32, 4] * 64, 32),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_call_eager_equals_fused(case):
    """Called directly (no capture), the device-planned call gives the same
    bits as lora_sgmv_fused on the same request-order batch (token_rows)."""
    import torch
    import lora_adapter_batching_amd as L
    name, T, h_in, h_out, ranks, max_rank = case
    prob = _problem(3, T, h_in, h_out, ranks)
    tb = _Tables(prob, max_rank)
    x = dev_bf16(prob.x)
    ids = torch.from_numpy(prob.token_ids.copy()).cuda()
    y_graph = dev_bf16(prob.y0)
    ws = L.new_workspace_graph(tb.ga, T)
    _say(f"graph call eager {name}")
    L.sgmv_fused_graph(x, tb.ga, ids, y_graph, ws)
    perm, st, ad = L.segments_from_ids(prob.token_ids, prob.N)
    rows = torch.from_numpy(perm.copy()).cuda()
    ad_h = L.Adapters(tb.A, tb.B, prob.ranks, prob.scales, h_in, h_out)
    sg = L.Segments(st, ad, rows)
    y_fused = dev_bf16(prob.y0)
    _say(f"lora_sgmv_fused {name}")
    L.sgmv_fused(x, ad_h, sg, y_fused, None, L.new_workspace(L.OP_FUSED, ad_h, sg))
    torch.cuda.synchronize()
    assert torch.equal(y_graph.view(torch.int16), y_fused.view(torch.int16))
    e = rel_err(to_f64(y_graph), tb.oracle_y(prob.x, prob.y0, prob.token_ids))
    assert e <= BF16_TOL, f"y rel err {e:.3e}"


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_graph_capture_replays_with_new_ids_weights_and_tables(case):
    """One capture, several replays; before each replay the ids, weights
    (in place), a scale, a rank and two table entries (re-pointed to weights
    of another rank) change in device memory. Eager library work runs
    between the replays. Every replay matches the oracle on its own inputs."""
    import torch
    import lora_adapter_batching_amd as L
    name, T, h_in, h_out, ranks, max_rank = case
    prob = _problem(5, T, h_in, h_out, ranks)
    N = prob.N
    tb = _Tables(prob, max_rank)
    x = dev_bf16(prob.x)
    ids = torch.from_numpy(prob.token_ids.copy()).cuda()
    y = dev_bf16(prob.y0)
    ws = L.new_workspace_graph(tb.ga, T)
    # eager work between replays: a plain fused call on buffers of its own
    side = _problem(6, 96, h_in, 256, [16, 8])
    sperm, sst, sad = L.segments_from_ids(side.token_ids, side.N)
    s_ad = L.Adapters([dev_bf16(a) for a in side.A], [dev_bf16(b) for b in side.B], side.ranks, side.scales,
                      h_in, 256)
    s_sg = L.Segments(sst, sad)
    s_x = dev_bf16(side.x[sperm])
    s_ws = L.new_workspace(L.OP_FUSED, s_ad, s_sg)
    # warm-up outside the capture, then capture on torch's capture stream
    L.sgmv_fused_graph(x, tb.ga, ids, y, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say(f"capture {name}")
    with torch.cuda.graph(g):
        L.sgmv_fused_graph(x, tb.ga, ids, y, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    spare = []  # keeps re-pointed weights alive
    for rep in range(5):
        new_ids = prob.token_ids.copy()
        if rep == 1:
            new_ids = rng.integers(0, N, size=T).astype(np.int32)
            new_ids[rng.random(T) < 0.15] = -1
            new_ids[rng.random(T) < 0.05] = 99  # outside [0, N): no adapter
        elif rep == 2:
            # in-place weight update of adapter 0 and a new scale for adapter 1
            one = np.zeros(1, np.int32)
            a0 = make_custom(100 + rep, h_in, h_out, [int(tb.ranks[0])], ids=one).A[0]
            b0 = make_custom(200 + rep, h_in, h_out, [int(tb.ranks[0])], ids=one).B[0]
            tb.A[0].copy_(dev_bf16(a0))
            tb.B[0].copy_(dev_bf16(b0))
            tb.A_bits[0], tb.B_bits[0] = a0, b0
            tb.scales[1] = 0.75
            tb.scales_dev[1] = 0.75
            new_ids = rng.integers(0, N, size=T).astype(np.int32)
        elif rep == 3:
            # re-point adapter N-1 to weights of another rank (<= max_rank)
            r_new = min(16 if int(tb.ranks[N - 1]) != 16 else 8, max_rank)
            w = make_custom(300 + rep, h_in, h_out, [r_new], ids=np.zeros(1, np.int32))
            A_new, B_new = dev_bf16(w.A[0]), dev_bf16(w.B[0])
            spare.append((A_new, B_new))
            tb.A_ptrs[N - 1] = A_new.data_ptr()
            tb.B_ptrs[N - 1] = B_new.data_ptr()
            tb.ranks[N - 1] = r_new
            tb.ranks_dev[N - 1] = r_new
            tb.A_bits[N - 1], tb.B_bits[N - 1] = w.A[0], w.B[0]
            new_ids = rng.integers(0, N, size=T).astype(np.int32)
        elif rep == 4:
            new_ids = np.full(T, N - 1, np.int32)  # one adapter carries the whole batch
        ids.copy_(torch.from_numpy(new_ids))
        y0 = make_custom(400 + rep, h_in, h_out, [8], ids=np.zeros(T, np.int32), y0=True).y0
        y.copy_(dev_bf16(y0))
        L.sgmv_fused(s_x, s_ad, s_sg, torch.zeros((96, 256), dtype=torch.bfloat16, device="cuda"), None, s_ws)
        torch.cuda.synchronize()
        _say(f"replay {rep} {name}")
        g.replay()
        torch.cuda.synchronize()
        ref = tb.oracle_y(prob.x, y0, new_ids)
        got = to_f64(y)
        e = rel_err(got, ref)
        assert e <= BF16_TOL, f"replay {rep}: y rel err {e:.3e}"
        # rows without an active adapter are left exactly as they were
        inactive = np.array([not (0 <= i < N and tb.ranks[i] > 0) for i in new_ids])
        assert np.array_equal(got[inactive], oracle.widen(y0)[inactive])



def test_graph_of_several_steps_shares_workspaces():
    """Two decode steps of two projections captured in one graph (four
    device-planned launches), each projection's workspace used by both
    steps, all calls reading one device id array. Replayed with new ids and
    fresh outputs; every output matches the oracle on every replay."""
    import torch
    import lora_adapter_batching_amd as L
    T = 256
    rng = np.random.default_rng(21)
    ids0 = rng.integers(0, 8, size=T).astype(np.int32)
    shapes = [(2560, 2560, [32] * 8, 32), (1024, 4096, [8, 16, 0, 64, 32, 16, 8, 24], 64)]
    projs, tables, wss = [], [], []
    for j, (h_in, h_out, ranks, max_rank) in enumerate(shapes):
        prob = make_custom(30 + j, h_in, h_out, ranks, scales="random", ids=ids0, y0=True)
        projs.append(prob)
        tables.append(_Tables(prob, max_rank))
        wss.append(L.new_workspace_graph(tables[-1].ga, T))
    ids = torch.from_numpy(ids0.copy()).cuda()
    steps = []  # (projection, x bits, x, y)
    for s in range(2):
        for j, prob in enumerate(projs):
            xb = make_custom(40 + 2 * s + j, prob.h_in, prob.h_out, [8], ids=np.zeros(T, np.int32)).x
            steps.append((j, xb, dev_bf16(xb), torch.zeros((T, prob.h_out), dtype=torch.bfloat16, device="cuda")))
    for j, xb, x, y in steps:  # warm-up outside the capture
        L.sgmv_fused_graph(x, tables[j].ga, ids, y, wss[j])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("capture two steps x two projections")
    with torch.cuda.graph(g):
        for j, xb, x, y in steps:
            L.sgmv_fused_graph(x, tables[j].ga, ids, y, wss[j])
    torch.cuda.synchronize()
    for rep in range(3):
        new_ids = ids0 if rep == 0 else rng.integers(-1, 9, size=T).astype(np.int32)
        ids.copy_(torch.from_numpy(new_ids))
        y0s = []
        for k, (j, xb, x, y) in enumerate(steps):
            y0 = make_custom(500 + 10 * rep + k, projs[j].h_in, projs[j].h_out, [8], ids=np.zeros(T, np.int32),
                             y0=True).y0
            y.copy_(dev_bf16(y0))
            y0s.append(y0)
        torch.cuda.synchronize()
        _say(f"replay {rep} of the two-step graph")
        g.replay()
        torch.cuda.synchronize()
        for k, (j, xb, x, y) in enumerate(steps):
            e = rel_err(to_f64(y), tables[j].oracle_y(xb, y0s[k], new_ids))
            assert e <= BF16_TOL, f"replay {rep} call {k}: y rel err {e:.3e}"

def test_double_buffered_tables_update_during_decode():
    """Two table sets differ in one adapter's weight buffers. A decode on
    stream 1 reads set 0 while stream 2 overwrites the other buffer (set 1's)
    with the updated weights; stream 1 then decodes with set 1 after an
    event. Each result matches the oracle on the weights its table pointed
    to."""
    import torch
    import lora_adapter_batching_amd as L
    T, h_in, h_out, N, k = 256, 2560, 2560, 8, 3
    prob = _problem(21, T, h_in, h_out, [32] * N)
    t0 = _Tables(prob, 32)
    t1 = _Tables(prob, 32)
    # set 1 shares every buffer with set 0 except adapter k's, which starts as garbage
    upd = make_custom(22, h_in, h_out, [32], ids=np.zeros(1, np.int32))
    A_buf = torch.full_like(t0.A[k], float("nan"))
    B_buf = torch.full_like(t0.B[k], float("nan"))
    for i in range(N):
        if i != k:
            t1.A_ptrs[i] = t0.A[i].data_ptr()
            t1.B_ptrs[i] = t0.B[i].data_ptr()
    t1.A_ptrs[k] = A_buf.data_ptr()
    t1.B_ptrs[k] = B_buf.data_ptr()
    t1.A_bits[k], t1.B_bits[k] = upd.A[0], upd.B[0]
    A_new, B_new = dev_bf16(upd.A[0]), dev_bf16(upd.B[0])
    x = dev_bf16(prob.x)
    ids = torch.from_numpy(prob.token_ids.copy()).cuda()
    y_old = dev_bf16(prob.y0)
    y_new = dev_bf16(prob.y0)
    ws0 = L.new_workspace_graph(t0.ga, T)
    ws1 = L.new_workspace_graph(t1.ga, T)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    _say("decode on stream 1 with table set 0, weight update on stream 2")
    with torch.cuda.stream(s1):
        for _ in range(3):  # keep stream 1 busy while stream 2 writes
            y_old.copy_(dev_bf16(prob.y0))
            L.sgmv_fused_graph(x, t0.ga, ids, y_old, ws0)
    with torch.cuda.stream(s2):
        A_buf.copy_(A_new)
        B_buf.copy_(B_new)
        ev = torch.cuda.Event()
        ev.record()
    s1.wait_event(ev)
    with torch.cuda.stream(s1):
        L.sgmv_fused_graph(x, t1.ga, ids, y_new, ws1)
    torch.cuda.synchronize()
    e0 = rel_err(to_f64(y_old), t0.oracle_y(prob.x, prob.y0, prob.token_ids))
    e1 = rel_err(to_f64(y_new), t1.oracle_y(prob.x, prob.y0, prob.token_ids))
    assert e0 <= BF16_TOL, f"set 0: y rel err {e0:.3e}"
    assert e1 <= BF16_TOL, f"set 1: y rel err {e1:.3e}"
    # the update changed adapter k's rows and only those
    m = prob.token_ids == k
    d = to_f64(y_old) != to_f64(y_new)
    assert np.any(d[m]) and not np.any(d[~m])


def test_one_workspace_serves_both_planners():
    """One workspace, sized for the largest batch, serves calls of several
    sizes in turn, planned inside the launch (<= 1024 tokens) or by the plan
    kernel (more): the epoch keeps every call's hand-off distinct across
    both kinds, and each call gives the same bits as lora_sgmv_fused."""
    import torch
    import lora_adapter_batching_amd as L
    h_in, h_out, ranks = 2048, 2048, [32] * 6 + [16] * 2
    T_max = 1400
    big = _problem(31, T_max, h_in, h_out, ranks)
    tb = _Tables(big, 32)
    x = dev_bf16(big.x)
    ws = L.new_workspace_graph(tb.ga, T_max)
    ad_h = L.Adapters(tb.A, tb.B, big.ranks, big.scales, h_in, h_out)
    rng = np.random.default_rng(32)
    for T in (256, 1400, 96, 1024, 1400, 256):
        need = L.workspace_size_graph(tb.ga, T)
        assert need <= ws.numel(), (T, need, ws.numel())
        ids_h = rng.integers(0, big.N, size=T).astype(np.int32)
        ids = torch.from_numpy(ids_h).cuda()
        y0 = dev_bf16(big.y0[:T])
        y_graph = y0.clone()
        _say(f"shared workspace, {T} tokens")
        L.sgmv_fused_graph(x[:T], tb.ga, ids, y_graph, ws)
        perm, st, ad = L.segments_from_ids(ids_h, big.N)
        sg = L.Segments(st, ad, torch.from_numpy(perm.copy()).cuda())
        y_fused = y0.clone()
        L.sgmv_fused(x[:T], ad_h, sg, y_fused, None, L.new_workspace(L.OP_FUSED, ad_h, sg))
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int16), y_fused.view(torch.int16)), T
    e = rel_err(to_f64(y_graph), tb.oracle_y(big.x[:T], big.y0[:T], ids_h))
    assert e <= BF16_TOL, f"y rel err {e:.3e}"


# Batches far above the 1024 tokens a launch plans by itself, in the layouts
# the planner picks for them: the medium split (a prefill-sized batch; an
# MLP-up batch with ranks to 128) and one on-chip item per tile (more tiles
# than resident workgroups).
BIG = [
    ("prefill_8192tok_4096", 8192, 4096, 4096, [16] * 8, 16),
    ("mlp_up_4096tok_r8_128", 4096, 4096, 14336, [8, 16, 32, 64, 128, 0, 32, 16] * 4, 128),
    ("on_chip_20000tok", 20000, 1024, 1024, [8, 16, 32, 64] * 4, 64),
]


@pytest.mark.parametrize("case", BIG, ids=[c[0] for c in BIG])
def test_graph_call_large_batches(case):
    """Large request-order batches through the plan kernel: the eager call
    gives the same bits as lora_sgmv_fused and matches the oracle; a replay
    of its capture on new ids (some -1) matches the oracle too."""
    import torch
    import lora_adapter_batching_amd as L
    name, T, h_in, h_out, ranks, max_rank = case
    prob = _problem(41, T, h_in, h_out, ranks)
    tb = _Tables(prob, max_rank)
    x = dev_bf16(prob.x)
    ids = torch.from_numpy(prob.token_ids.copy()).cuda()
    y = dev_bf16(prob.y0)
    ws = L.new_workspace_graph(tb.ga, T)
    _say(f"graph call eager {name}")
    L.sgmv_fused_graph(x, tb.ga, ids, y, ws)
    perm, st, ad = L.segments_from_ids(prob.token_ids, prob.N)
    ad_h = L.Adapters(tb.A, tb.B, prob.ranks, prob.scales, h_in, h_out)
    sg = L.Segments(st, ad, torch.from_numpy(perm.copy()).cuda())
    y_fused = dev_bf16(prob.y0)
    _say(f"lora_sgmv_fused {name}")
    L.sgmv_fused(x, ad_h, sg, y_fused, None, L.new_workspace(L.OP_FUSED, ad_h, sg))
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_fused.view(torch.int16))
    e = rel_err(to_f64(y), tb.oracle_y(prob.x, prob.y0, prob.token_ids))
    assert e <= BF16_TOL, f"eager: y rel err {e:.3e}"
    g = torch.cuda.CUDAGraph()
    _say(f"capture {name}")
    with torch.cuda.graph(g):
        L.sgmv_fused_graph(x, tb.ga, ids, y, ws)
    rng = np.random.default_rng(42)
    new_ids = rng.integers(0, prob.N, size=T).astype(np.int32)
    new_ids[rng.random(T) < 0.1] = -1
    ids.copy_(torch.from_numpy(new_ids))
    y.copy_(dev_bf16(prob.y0))
    torch.cuda.synchronize()
    _say(f"replay {name}")
    g.replay()
    torch.cuda.synchronize()
    got = to_f64(y)
    e = rel_err(got, tb.oracle_y(prob.x, prob.y0, new_ids))
    assert e <= BF16_TOL, f"replay: y rel err {e:.3e}"
    inactive = np.array([not (0 <= i < prob.N and tb.ranks[i] > 0) for i in new_ids])
    assert np.array_equal(got[inactive], oracle.widen(prob.y0)[inactive])


# (T, h_in, h_out, number of adapters): widths multiples of 8 but not of 32,
# token counts on both sides of the 1024 the fused launch plans by itself
FUZZ = [(2, 72, 200, 3), (33, 264, 136, 1), (200, 520, 1032, 40), (511, 200, 264, 256), (1024, 1032, 520, 17),
        (1025, 136, 264, 5), (1900, 264, 1032, 64), (700, 2056, 72, 9)]


@pytest.mark.parametrize("case", range(len(FUZZ)))
def test_graph_call_random_shapes(case):
    """Seeded random batches through the device-planned call, eagerly and
    from a replayed capture, against the fp64 oracle: mixed ranks 0..128
    under a random max_rank, ids -1 and past N, unused adapters."""
    import torch
    import lora_adapter_batching_amd as L
    T, h_in, h_out, N = FUZZ[case]
    rng = np.random.default_rng(1300 + case)
    ranks = [int(r) for r in rng.choice([0, 1, 4, 8, 12, 16, 24, 32, 40, 64, 96, 128], size=N)]
    if max(ranks) == 0:
        ranks[0] = 8
    max_rank = int(min(128, max(ranks) + int(rng.integers(0, 16))))
    ids = rng.integers(-1, N + 2, size=T).astype(np.int32)
    if N > 2:
        ids[ids == 1] = 0  # an adapter without tokens
    prob = make_custom(1350 + case, h_in, h_out, ranks, scales="random", ids=ids, y0=True)
    tb = _Tables(prob, max_rank)
    x = dev_bf16(prob.x)
    idt = torch.from_numpy(ids.copy()).cuda()
    y = dev_bf16(prob.y0)
    ws = L.new_workspace_graph(tb.ga, T)
    _say(f"graph fuzz {case}: T={T} {h_in}->{h_out} N={N} max_rank={max_rank}")
    L.sgmv_fused_graph(x, tb.ga, idt, y, ws)
    torch.cuda.synchronize()
    ref = tb.oracle_y(prob.x, prob.y0, ids)
    got = to_f64(y)
    assert rel_err(got, ref) <= BF16_TOL, "eager call"
    inactive = np.array([not (0 <= i < N and ranks[i] > 0) for i in ids])
    assert np.array_equal(got[inactive], oracle.widen(prob.y0)[inactive])
    # the same call replayed from a capture, on new ids
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.sgmv_fused_graph(x, tb.ga, idt, y, ws)
    torch.cuda.synchronize()
    for rep in range(2):
        ids2 = rng.integers(-1, N + 2, size=T).astype(np.int32)
        idt.copy_(torch.from_numpy(ids2))
        y.copy_(dev_bf16(prob.y0))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e = rel_err(to_f64(y), tb.oracle_y(prob.x, prob.y0, ids2))
        assert e <= BF16_TOL, f"replay {rep}: y rel err {e:.3e}"
