"""CPU checks of the segment scheduler (no GPU).

The library's planner turns segments x ranks x shapes into work items; the
internal inspection entry (csrc/lora_inspect.h) runs exactly that planner
with stand-in device addresses and lists every workgroup of every launch a
call would make. These tests check the plan itself:

- coverage: every (position, output column) of an active segment is expanded
  exactly once, every shrink reduction range [0, K) is covered exactly once
  per tile, and skipped segments (adapter -1, rank 0, no tokens) get no item;
- ownership of the weight gradients: each adapter's tokens are walked exactly
  once over its jobs, each job's dA and dB columns are owned by exactly one
  item, token-range parts are summed by exactly one reduce pass;
- determinism: the same inputs give the same plan, bit for bit;
- balance over heterogeneous adapters ("Technische Samenvatting: PLoRA"
  (gist.science), "Kernelontwerp": load balancing over adapters of
  different ranks and lengths): on the MLP-up workload with ranks 8..128 and
  Zipf-popular adapters, the predicted per-CU cost of an in-order dispatch
  stays within 1.15x of the mean.
"""
import ctypes

import numpy as np
import pytest

import lora_adapter_batching_amd as L
from lora_adapter_batching_amd import binding as B
from workloads import make_meta

FAKE = 1 << 20


class _HostAdapters:
    """lora_adapters_t with stand-in device tables (never dereferenced)."""

    def __init__(self, ranks, h_in, h_out, scales=None, host_tables=True, base=0):
        self.ranks = np.ascontiguousarray(ranks, np.int32)
        n = len(self.ranks)
        self.scales = np.ascontiguousarray(scales if scales is not None else [2.0] * n, np.float32)
        self.A_host = np.array([FAKE * (2 + 2 * i + base) for i in range(n)], np.uint64)
        self.B_host = np.array([FAKE * (3 + 2 * i + base) for i in range(n)], np.uint64)
        self._c = B.CAdapters(n, h_in, h_out, FAKE, FAKE, self.ranks.ctypes.data, self.scales.ctypes.data,
                              self.A_host.ctypes.data if host_tables else 0,
                              self.B_host.ctypes.data if host_tables else 0)
        self.h_in, self.h_out = h_in, h_out


def _segments_of(meta, token_rows=False):
    if meta.segmented:
        starts = np.concatenate([[0], np.cumsum(meta.seg_lens)]).astype(np.int32)
        adap = np.asarray(meta.seg_adapter, np.int32)
    else:
        _, starts, adap = L.segments_from_ids(meta.token_ids, meta.N)
    return L.Segments(starts, adap, FAKE if token_rows else None), starts, adap


def _active(starts, adap, ranks):
    """positions -> adapter for active segments (-1 elsewhere)."""
    T = int(starts[-1])
    a = np.full(T, -1, np.int64)
    for g in range(len(adap)):
        i = int(adap[g])
        if i >= 0 and ranks[i] > 0:
            a[starts[g]:starts[g + 1]] = i
    return a


def _fwd_items(items, kinds):
    f = items[items["phase"] == B.PHASE_FWD]
    return f[np.isin(f["kind"], kinds)]


def _check_expand_cover(items, a_pos, h_out, proj=0, launches=None):
    """Every (active position, column) covered exactly once by expand kinds."""
    T = len(a_pos)
    cover = np.zeros((T, h_out), np.int32)
    ex = _fwd_items(items, [1, 2, 3])
    ex = ex[ex["proj"] == proj]
    if launches is not None:
        ex = ex[np.isin(ex["launch"], launches)]
    for r in ex:
        assert 0 <= r["lo"] <= r["hi"] <= h_out
        assert 1 <= r["ntok"] <= 32
        p0, p1 = r["tok0"], r["tok0"] + r["ntok"]
        assert np.all(a_pos[p0:p1] == r["adapter"]), "an item spans positions of another adapter"
        cover[p0:p1, r["lo"]:r["hi"]] += 1
    act = a_pos >= 0
    assert np.all(cover[act] == 1), "active (position, column) not covered exactly once"
    assert np.all(cover[~act] == 0), "a skipped position got work"


def _check_shrink_cover(items, K, launches=None):
    """Per (launch, tile): the shrink parts cover [0, K) exactly once; the
    waiting expands of a tile find all of its parts in their own launch."""
    sh = _fwd_items(items, [0])
    if launches is not None:
        sh = sh[np.isin(sh["launch"], launches)]
    tiles = {}
    for r in sh:
        tiles.setdefault((int(r["launch"]), int(r["tile"])), []).append((int(r["lo"]), int(r["hi"])))
    for key, rngs in tiles.items():
        cov = np.zeros(K, np.int32)
        for lo, hi in rngs:
            assert 0 <= lo < hi <= K
            cov[lo:hi] += 1
        assert np.all(cov == 1), f"shrink parts of {key} do not cover [0, K) once"
    wait = _fwd_items(items, [3])
    for r in wait:
        assert (int(r["launch"]), int(r["tile"])) in tiles, "waiting expand without shrink parts"
    return tiles


def _plan(op, ads, sg, options=0, cus=256, xccs=8):
    items, ranges = B.inspect_plan(op, ads, sg, options, cus, xccs)
    assert len(items) > 0 or op == B.OP_EXPAND
    return items, ranges


CASES = [("tiny", None), ("decode", "q"), ("decode", "gate_up"), ("prefill", None), ("hetero", None)]


@pytest.mark.parametrize("name,proj", CASES)
@pytest.mark.parametrize("xccs", [8, 1])
def test_fused_plan_covers_every_output_once(name, proj, xccs):
    m = make_meta(name, proj=proj or "gate_up")
    sg, st, ad = _segments_of(m)
    a = _HostAdapters(m.ranks, m.h_in, m.h_out)
    items, _ = _plan(B.OP_FUSED, a, sg, xccs=xccs)
    assert set(np.unique(items["phase"])) == {B.PHASE_FWD}
    a_pos = _active(st, ad, m.ranks)
    _check_expand_cover(items, a_pos, m.h_out)
    _check_shrink_cover(items, m.h_in)
    # one launch per call for these batches (at most 128 segments)
    assert len(np.unique(items["launch"])) == 1
    # every workgroup of the grid is listed once
    assert len(items) == int(items["grid"][0])
    assert np.array_equal(np.sort(items["block"]), np.arange(len(items)))
    if name == "decode":
        busy = items[items["kind"] >= 0]
        if xccs == 8 or proj == "gate_up":
            assert np.all(busy["mode"] == 3)  # split shrink, parts handed to the expands
        if proj == "q" and xccs == 8:
            # small batch on 8 XCDs: all items of tile g run on XCD g % 8
            assert np.all(busy["block"] % 8 == busy["tile"] % 8)
        if proj == "gate_up":
            # an expand-heavy small batch spreads every tile's items over all
            # XCDs, parts of at most 320 columns (8 per tile at h_in 2560)
            assert any(len(np.unique(busy[busy["tile"] == g]["block"] % 8)) == 8 for g in np.unique(busy["tile"]))
            assert int(items["part"][0]) == 8


def test_fused_plan_many_segments_and_edge_cases():
    rng = np.random.default_rng(5)
    for trial in range(12):
        N = int(rng.integers(1, 40))
        ranks = rng.choice([0, 1, 8, 12, 16, 24, 32, 40, 64, 100, 128], size=N).astype(np.int32)
        T = int(rng.choice([0, 1, 31, 33, 257, 1000, 5000, 20000]))
        ids = rng.integers(-1, N, size=T).astype(np.int32)
        h_in = int(rng.choice([8, 72, 256, 2560, 4096]))
        h_out = int(rng.choice([8, 40, 256, 1000, 4104]))
        _, st, ad = L.segments_from_ids(ids, N)
        # split some segments in two, so adapters repeat and segments exceed 128
        lens = np.diff(st)
        seg_l, seg_a = [], []
        for g in range(len(ad)):
            n = int(lens[g])
            if n > 3 and rng.random() < 0.5:
                k = int(rng.integers(1, n))
                seg_l += [k, n - k]
                seg_a += [int(ad[g])] * 2
            else:
                seg_l.append(n)
                seg_a.append(int(ad[g]))
        starts = np.concatenate([[0], np.cumsum(seg_l)]).astype(np.int32)
        sg = L.Segments(starts, np.array(seg_a, np.int32))
        a = _HostAdapters(ranks, h_in, h_out, host_tables=bool(trial % 2))
        items, _ = B.inspect_plan(B.OP_FUSED, a, sg, B.INSPECT_WITH_U)
        a_pos = _active(starts, np.array(seg_a), ranks)
        if not np.any(a_pos >= 0):
            assert len(items) == 0
            continue
        _check_expand_cover(items, a_pos, h_out)
        _check_shrink_cover(items, h_in)
        # no item is planned for a rank-0 adapter, an id -1 or an empty segment
        busy = items[items["kind"] >= 0]
        assert np.all(ranks[busy["adapter"]] > 0)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "hetero"])
def test_shrink_and_expand_plans_cover_once(name):
    m = make_meta(name)
    sg, st, ad = _segments_of(m)
    a = _HostAdapters(m.ranks, m.h_in, m.h_out)
    a_pos = _active(st, ad, m.ranks)
    items, _ = _plan(B.OP_SHRINK, a, sg)
    assert np.all(items[items["kind"] >= 0]["kind"] == 0)
    tiles = _check_shrink_cover(items, m.h_in)
    covered = np.zeros(len(a_pos), np.int32)
    seen = set()
    for r in _fwd_items(items, [0]):
        key = (int(r["launch"]), int(r["tile"]))
        if key not in seen:
            seen.add(key)
            covered[r["tok0"]:r["tok0"] + r["ntok"]] += 1
    assert np.all(covered[a_pos >= 0] == 1) and np.all(covered[a_pos < 0] == 0)
    assert len(seen) == len(tiles)
    items, _ = _plan(B.OP_EXPAND, a, sg)
    assert np.all(items[items["kind"] >= 0]["kind"] == 1)
    _check_expand_cover(items, a_pos, m.h_out)


def test_multi_projection_plan_covers_each_projection():
    m = make_meta("decode")
    sg, st, ad = _segments_of(m)
    widths = [4096, 1024, 1024]
    ads = [_HostAdapters(np.array([32, 0, 16, 32, 8, 32, 32, 24][:m.N]) if p == 1 else m.ranks, m.h_in, w,
                         base=100 * p) for p, w in enumerate(widths)]
    items, _ = _plan(B.OP_FUSED, ads, sg)
    for p, w in enumerate(widths):
        _check_expand_cover(items, _active(st, ad, ads[p].ranks), w, proj=p)
    _check_shrink_cover(items, m.h_in)


def _check_backward(items, ranges, m, starts, adap, accumulate, with_dx):
    ranks = m.ranks
    a_pos = _active(starts, adap, ranks)
    # du / dx passes: forward-style launches over dy (K = h_out) into dx (N = h_in)
    fwd_launches = np.unique(items[items["phase"] == B.PHASE_FWD]["launch"])
    dudx = [l for l in fwd_launches if np.any(_fwd_items(items, [0, 2, 3])["launch"] == l)]
    if with_dx:
        _check_expand_cover(items, a_pos, m.h_in, launches=[l for l in dudx if np.any(
            _fwd_items(items, [2, 3])["launch"] == l)])
    # weight gradients
    wg = items[items["phase"] == B.PHASE_WGRAD]
    tok_cover = np.zeros(len(a_pos), np.int32)
    jobs = {}
    for r in wg:
        jobs.setdefault((int(r["launch"]), int(r["tile"])), []).append(r)
    parts = {}
    zero_fill = set()
    for key, rs in jobs.items():
        r0 = rs[0]
        i = int(r0["adapter"])
        assert ranks[i] > 0, "weight-gradient job for a rank-0 adapter"
        db = np.zeros(m.h_out, np.int32)
        da = np.zeros(m.h_in, np.int32)
        for r in rs:
            assert r["adapter"] == i and r["tok0"] == r0["tok0"] and r["ntok"] == r0["ntok"]
            (db if r["kind"] == 0 else da)[r["lo"]:r["hi"]] += 1
        assert np.all(db == 1) and np.all(da == 1), "a dA/dB column chunk is not owned by exactly one item"
        rg = ranges[r0["tok0"]:r0["tok0"] + r0["ntok"]]
        if len(rg) == 0 or rg[:, 1].sum() == 0:
            zero_fill.add(i)
        for p0, n in rg:
            assert np.all(a_pos[p0:p0 + n] == i), "a job walks tokens of another adapter"
            tok_cover[p0:p0 + n] += 1
        if r0["part"] >= 0:
            parts.setdefault(i, []).append(int(r0["part"]))
    assert np.all(tok_cover[a_pos >= 0] == 1), "an adapter's tokens are not walked exactly once"
    assert np.all(tok_cover[a_pos < 0] == 0)
    with_tokens = set(int(v) for v in np.unique(a_pos[a_pos >= 0]))
    expect_zero = set() if accumulate else {i for i in range(m.N) if ranks[i] > 0} - with_tokens
    assert zero_fill == expect_zero
    # token-range parts: one reduce over exactly the adapter's slots
    red = items[items["phase"] == B.PHASE_REDUCE]
    for i, slots in parts.items():
        rr = red[red["adapter"] == i]
        assert len(rr) > 0
        n_all = (m.h_in + m.h_out) * int(ranks[i])
        cov = np.zeros(n_all, np.int32)
        for r in rr:
            cov[r["lo"]:r["hi"]] += 1
            assert r["part"] == min(slots) and r["aux"] == len(slots)
        assert np.all(cov == 1)
        assert sorted(slots) == list(range(min(slots), min(slots) + len(slots)))


@pytest.mark.parametrize("name", ["tiny", "prefill", "hetero", "train"])
@pytest.mark.parametrize("options", [B.INSPECT_WITH_U | B.INSPECT_WITH_DX, B.INSPECT_WITH_DX | B.INSPECT_ACCUMULATE,
                                     0])
def test_backward_plan_ownership(name, options):
    m = make_meta(name)
    sg, st, ad = _segments_of(m)
    a = _HostAdapters(m.ranks, m.h_in, m.h_out)
    items, ranges = _plan(B.OP_BACKWARD, a, sg, options)
    _check_backward(items, ranges, m, st, ad, bool(options & B.INSPECT_ACCUMULATE),
                    bool(options & B.INSPECT_WITH_DX))


def test_backward_plan_splits_few_long_adapters():
    """One or two adapters carrying all tokens: the planner cuts their token
    walks into parts (partial slots plus a reduce), and ownership holds."""
    for n_ad, T in ((1, 2048), (2, 4096), (3, 8192)):
        lens = np.full(n_ad, T // n_ad, np.int32)
        sa = np.arange(n_ad, dtype=np.int32)
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ranks = np.array([16, 64, 8][:n_ad] + [32], np.int32)  # plus an adapter with no tokens
        a = _HostAdapters(ranks, 3584, 3584)
        sg = L.Segments(starts, sa)
        items, ranges = _plan(B.OP_BACKWARD, a, sg, B.INSPECT_WITH_U | B.INSPECT_WITH_DX)
        assert np.any(items["phase"] == B.PHASE_REDUCE)

        class M:
            pass
        m = M()
        m.ranks, m.N, m.h_in, m.h_out = ranks, len(ranks), 3584, 3584
        _check_backward(items, ranges, m, starts, sa, False, True)


@pytest.mark.parametrize("name", ["decode", "prefill", "hetero", "train"])
def test_plans_are_bit_identical_run_to_run(name):
    m = make_meta(name)
    sg, st, ad = _segments_of(m)
    a = _HostAdapters(m.ranks, m.h_in, m.h_out)
    op = B.OP_BACKWARD if name == "train" else B.OP_FUSED
    i1, r1 = _plan(op, a, sg, B.INSPECT_WITH_DX)
    i2, r2 = _plan(op, a, sg, B.INSPECT_WITH_DX)
    assert i1.tobytes() == i2.tobytes() and r1.tobytes() == r2.tobytes()


def _item_cost(r, K, widths):
    """Bytes an item moves (tile rows of x or y, its share of the weights)."""
    n = int(r["ntok"])
    w = int(r["hi"] - r["lo"])
    rank = int(r["rank"])
    if r["kind"] == 0:
        return 2 * n * w + 2 * rank * w
    if r["kind"] == 2:
        return 2 * n * K + 2 * rank * K + 4 * n * w + 2 * rank * w
    return 4 * n * w + 2 * rank * w


def _per_cu_cost(items, K, widths, cus=256, xccs=8, slots=2):
    """In-order dispatch: workgroup b goes to XCD b % xccs, there to the
    resident slot that frees first; a CU's cost is the sum over its slots."""
    per_xcd = cus // xccs
    load = np.zeros((xccs, per_xcd * slots))
    for r in items[np.argsort(items["block"], kind="stable")]:
        if r["kind"] < 0:
            continue
        x = int(r["block"]) % xccs
        s = int(np.argmin(load[x]))
        load[x, s] += _item_cost(r, K, widths)
    return load.reshape(xccs, per_xcd, slots).sum(axis=2).ravel()


def test_hetero_plan_balance_within_bound():
    m = make_meta("hetero")
    sg, st, ad = _segments_of(m)
    a = _HostAdapters(m.ranks, m.h_in, m.h_out)
    items, _ = _plan(B.OP_FUSED, a, sg)
    cu = _per_cu_cost(items, m.h_in, [m.h_out])
    ratio = float(cu.max() / cu.mean())
    assert ratio <= 1.15, f"max/mean predicted per-CU cost {ratio:.3f}"


def test_backward_plan_without_tokens_only_zero_fills():
    """A batch with no active tokens (every id -1, or only rank-0 adapters):
    the backward plans only the zero-gradient items of adapters with a rank
    (overwrite mode), and nothing at all in accumulate mode; no launch of
    the plan has an empty grid."""
    ranks = np.array([8, 0, 32], np.int32)
    a = _HostAdapters(ranks, 256, 128)
    for starts, adap in (([0, 5], [-1]), ([0, 4, 9], [1, -1])):
        sg = L.Segments(np.array(starts, np.int32), np.array(adap, np.int32))
        items, ranges = B.inspect_plan(B.OP_BACKWARD, a, sg, B.INSPECT_WITH_DX)
        assert set(np.unique(items["phase"])) == {B.PHASE_WGRAD}
        assert sorted(set(int(v) for v in items["adapter"])) == [0, 2]
        assert len(ranges) == 0
        items, _ = B.inspect_plan(B.OP_BACKWARD, a, sg, B.INSPECT_WITH_DX | B.INSPECT_ACCUMULATE)
        assert len(items) == 0


GRAPH_CASES = [
    # (adapters, h_in, h_out, max_rank, tokens): decode q and gate_up, many small adapters, odd widths
    (8, 2560, 2560, 32, 256),
    (8, 2560, 19456, 32, 256),
    (13, 2048, 1024, 16, 1024),
    (40, 1024, 1536, 128, 700),
    (256, 512, 512, 4, 512),
    (3, 200, 264, 64, 37),
    (8, 1024, 2048, 32, 1500),  # more tokens than a launch plans by itself: the plan kernel's tiles
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=[f"{c[0]}ad_{c[1]}x{c[2]}_r{c[3]}_{c[4]}tok" for c in GRAPH_CASES])
@pytest.mark.parametrize("xccs", [8, 1])
def test_device_planned_layout_covers_every_tile_count(case, xccs):
    """A device-planned launch of up to 1024 tokens lays its grid out for the
    most tiles the ids could need; its workgroups then re-lay the split
    layout out for the tiles the batch has. For every possible tile count:
    each tile's shrink parts cover [0, h_in) once, its expand items cover
    [0, h_out) once, no item names a tile past the count, and every item
    lies inside the grid (the listing has exactly one record per
    workgroup)."""
    N, h_in, h_out, max_rank, T = case
    max_tiles = -(-T // 32) + min(N, T)
    grids = set()
    for tiles in range(0, max_tiles + 1):
        items = B.inspect_graph(N, h_in, h_out, max_rank, T, tiles, cus=256, xccs=xccs)
        assert np.any(items["phase"] == B.PHASE_PLAN) == (T > 1024)
        f = items[items["phase"] == B.PHASE_FWD]
        assert len(f) == int(f["grid"][0]), "one record per workgroup"
        assert np.array_equal(np.sort(f["block"]), np.arange(len(f)))
        grids.add(int(f["grid"][0]))
        busy = f[f["kind"] >= 0]
        assert np.all(busy["tile"] < tiles), "an item past the batch's tiles"
        split = np.any(busy["kind"] == 0)
        for g in range(tiles):
            mine = busy[busy["tile"] == g]
            if split:
                cov = np.zeros(h_in, np.int32)
                for r in mine[mine["kind"] == 0]:
                    cov[r["lo"]:r["hi"]] += 1
                assert np.all(cov == 1), f"tiles={tiles}: shrink parts of tile {g}"
            cov = np.zeros(h_out, np.int32)
            for r in mine[mine["kind"] != 0]:
                cov[r["lo"]:r["hi"]] += 1
            assert np.all(cov == 1), f"tiles={tiles}: expand columns of tile {g}"
    assert len(grids) == 1, "the grid depends only on the token count"


GRAPH_BIG = [
    # (adapters, h_in, h_out, max_rank, tokens): the large batches of the GPU
    # graph tests (medium split twice, then one on-chip item per tile)
    (8, 4096, 4096, 16, 8192),
    (32, 4096, 14336, 128, 4096),
    (16, 1024, 1024, 64, 20000),
    (256, 264, 512, 32, 2048),  # the widest count scan, through the plan kernel
]


@pytest.mark.parametrize("case", GRAPH_BIG, ids=[f"{c[0]}ad_{c[1]}x{c[2]}_r{c[3]}_{c[4]}tok" for c in GRAPH_BIG])
def test_device_planned_large_batches_cover_every_tile(case):
    """Above 1024 tokens the plan kernel runs first and the fused launch is
    laid out for the most tiles the ids could need; a tile past the batch's
    count has no work (its workgroups return). For a few tile counts: each
    tile's shrink parts cover [0, h_in) once and its expand items [0, h_out)
    once, every item lies inside the grid, and the grid does not depend on
    the tile count."""
    N, h_in, h_out, max_rank, T = case
    max_tiles = -(-T // 32) + min(N, T)
    grids = set()
    for tiles in sorted({1, max_tiles // 3, max_tiles - 1, max_tiles}):
        items = B.inspect_graph(N, h_in, h_out, max_rank, T, tiles, cus=256, xccs=8)
        assert np.any(items["phase"] == B.PHASE_PLAN)
        f = items[items["phase"] == B.PHASE_FWD]
        assert len(f) == int(f["grid"][0]), "one record per workgroup"
        assert np.array_equal(np.sort(f["block"]), np.arange(len(f)))
        grids.add(int(f["grid"][0]))
        busy = f[f["kind"] >= 0]
        assert np.all(busy["tile"] < tiles), "an item past the batch's tiles"
        parts = busy[busy["kind"] == 0]
        if len(parts):
            cov = np.zeros((tiles, h_in + 1), np.int32)
            np.add.at(cov, (parts["tile"], parts["lo"]), 1)
            np.add.at(cov, (parts["tile"], parts["hi"]), -1)
            assert np.all(np.cumsum(cov, axis=1)[:, :h_in] == 1), f"tiles={tiles}: shrink parts"
        ex = busy[busy["kind"] != 0]
        cov = np.zeros((tiles, h_out + 1), np.int32)
        np.add.at(cov, (ex["tile"], ex["lo"]), 1)
        np.add.at(cov, (ex["tile"], ex["hi"]), -1)
        assert np.all(np.cumsum(cov, axis=1)[:, :h_out] == 1), f"tiles={tiles}: expand columns"
    assert len(grids) == 1, "the grid depends only on the token count"
