"""Benchmark of the multi-adapter LoRA (SGMV) hot path on one MI355X.

Headline step: one mixed-adapter decode step on Qwen3-4B-like projections --
256 tokens with adapter ids drawn uniformly from 8 resident rank-32 adapters
(scale 2), grouped into segments by the library's host bookkeeping, then one
fused shrink+expand launch per LoRA-wrapped projection: q (2560->2560),
o (2560->2560) and gate_up (2560->19456). Inputs are synthetic (seeded) and
resident in HBM; 16 copies of every tensor are rotated so that the 256 MB
Infinity Cache cannot serve a step from the previous one.

value = algorithmic bytes of the step / wall time per step (GB/s). Secondary
entries time the prefill, heterogeneous-rank and packed-training workloads
with HIP events (GB/s, TFLOP/s, fractions of the MI355X peaks).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu]
       python bench.py --sweep-adapters   (packed vs one-adapter-at-a-time calls, N = 1..32)
       python bench.py --only prefill|hetero|train [--reps R]   (one workload alone, for counter runs)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "SGMV decode HBM GB/s (% peak) + prefill/backward TFLOP/s (% MFMA peak)"
KERNEL = "sgmv_fwd_kernel"
WORKLOAD = "decode_qwen3_4b_q_o_gate_up_256tok_8x_r32"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Algorithmic work (what the method must move / compute; no padding)
# ---------------------------------------------------------------------------
def active_token_ranks(ranks, seg_starts, seg_adapter):
    """Per active token its rank (tokens of skipped segments excluded)."""
    out = []
    for g in range(len(seg_adapter)):
        a = int(seg_adapter[g])
        n = int(seg_starts[g + 1] - seg_starts[g])
        if a < 0 or n == 0 or ranks[a] == 0:
            continue
        out.append(np.full(n, int(ranks[a])))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def used_adapters(ranks, seg_starts, seg_adapter):
    s = set()
    for g in range(len(seg_adapter)):
        a = int(seg_adapter[g])
        if a >= 0 and seg_starts[g + 1] > seg_starts[g] and ranks[a] > 0:
            s.add(a)
    return sorted(s)


def fwd_work(h_in, h_out, ranks, seg_starts, seg_adapter, save_u=False):
    tr = active_token_ranks(ranks, seg_starts, seg_adapter)
    T = len(tr)
    w = sum(int(ranks[a]) * (h_in + h_out) for a in used_adapters(ranks, seg_starts, seg_adapter))
    bytes_ = 2 * T * h_in + 4 * T * h_out + 2 * w + (4 * int(tr.sum()) if save_u else 0)
    flops = 2 * (h_in + h_out) * int(tr.sum())
    return bytes_, flops


def shrink_work(h_in, ranks, seg_starts, seg_adapter):
    """x read, A_i read once, fp32 u written (rank columns only)."""
    tr = active_token_ranks(ranks, seg_starts, seg_adapter)
    w = sum(int(ranks[a]) * h_in for a in used_adapters(ranks, seg_starts, seg_adapter))
    return 2 * len(tr) * h_in + 2 * w + 4 * int(tr.sum()), 2 * h_in * int(tr.sum())


def expand_work(h_out, ranks, seg_starts, seg_adapter):
    """fp32 u read, B_i read once, y read and written."""
    tr = active_token_ranks(ranks, seg_starts, seg_adapter)
    w = sum(int(ranks[a]) * h_out for a in used_adapters(ranks, seg_starts, seg_adapter))
    return 4 * int(tr.sum()) + 2 * w + 4 * len(tr) * h_out, 2 * h_out * int(tr.sum())


def bwd_work(h_in, h_out, ranks, seg_starts, seg_adapter):
    tr = active_token_ranks(ranks, seg_starts, seg_adapter)
    T = len(tr)
    w = sum(int(ranks[a]) * (h_in + h_out) for a in used_adapters(ranks, seg_starts, seg_adapter))
    # dy, x read; dx read+write; u read; weights read; fp32 dA/dB written
    bytes_ = 2 * T * h_out + 2 * T * h_in + 4 * T * h_in + 4 * int(tr.sum()) + 2 * w + 4 * w
    flops = 4 * (h_in + h_out) * int(tr.sum())
    return bytes_, flops


# ---------------------------------------------------------------------------
def kernel_source_hash():
    """Hash of the library sources with comments and whitespace removed, so
    that counter summaries stay tied to the code they measured."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "lora_adapter_batching_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            src = open(os.path.join(csrc, f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            src = re.sub(r"//[^\n]*", "", src)
            h.update(re.sub(r"\s+", "", src).encode())
    return h.hexdigest()[:16]


def load_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<kernel>_<workload>.txt, 'key: value' lines), if it was
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", f"traffic_{KERNEL}_{workload}.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def dev_bf16(bits):
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda")


# ---------------------------------------------------------------------------
# Headline: decode step
# ---------------------------------------------------------------------------
class DecodeStep:
    """Pre-marshalled C-ABI calls for one decode step over a rotation set."""

    def __init__(self, projs, nsets, request_order=False, host_rows=False):
        import torch
        import lora_adapter_batching_amd as L
        from lora_adapter_batching_amd import binding as Bd
        self.lib = L.load()
        # request_order: x and y stay in the order the tokens arrived; every
        # step uploads its sorted-position -> row table (from the step's own
        # bookkeeping) and the kernels gather x rows and scatter y rows.
        # host_rows: the table is passed as the host copy instead, which the
        # small decode launches carry in their arguments (no upload)
        self.request_order = request_order
        self.host_rows = request_order and host_rows
        self.Bd = Bd
        p0 = projs["q"]
        self.ids = np.ascontiguousarray(p0.token_ids, np.int32)
        self.T, self.N = int(p0.T), int(p0.N)
        self.perm = np.zeros(self.T, np.int32)
        self.starts = np.zeros(self.N + 2, np.int32)
        self.adap = np.zeros(self.N + 1, np.int32)
        # bookkeeping once to size the workspace and to order the inputs
        perm, starts, adap = L.segments_from_ids(self.ids, self.N)
        self.seg = L.Segments(starts, adap)
        self.cseg = Bd.CSegments(self.T, self.N + 1, self.starts.ctypes.data, self.adap.ctypes.data, 0)
        self.names = ["q", "o", "gate_up"]
        self.sets = []
        self.keep = []
        if self.host_rows:
            self.cseg_host = Bd.CSegments(self.T, self.N + 1, self.starts.ctypes.data, self.adap.ctypes.data, 0,
                                          self.perm.ctypes.data)
        elif request_order:
            # one pinned host table, device table and event per rotation set:
            # a slot's host table is rewritten only after its last upload ended
            self.rows_host = [torch.zeros(self.T, dtype=torch.int32).pin_memory() for _ in range(nsets)]
            self.rows_dev = [torch.zeros(self.T, dtype=torch.int32, device="cuda") for _ in range(nsets)]
            self.rows_ev = [None] * nsets
            self.cseg_rows = [Bd.CSegments(self.T, self.N + 1, self.starts.ctypes.data, self.adap.ctypes.data,
                                           r.data_ptr()) for r in self.rows_dev]
        dev_inputs = {}
        for name in self.names:
            p = projs[name]
            xs = p.x if request_order else p.x[perm]
            dev_inputs[name] = (dev_bf16(xs), [dev_bf16(a) for a in p.A], [dev_bf16(b) for b in p.B])
        for s in range(nsets):
            calls = []
            for name in self.names:
                p = projs[name]
                x0, A0, B0 = dev_inputs[name]
                x = x0.clone()
                A = [a.clone() for a in A0]
                B = [b.clone() for b in B0]
                ad = L.Adapters(A, B, p.ranks, p.scales, p.h_in, p.h_out)
                y = torch.zeros((self.T, p.h_out), dtype=torch.bfloat16, device="cuda")
                ws = L.new_workspace(L.OP_FUSED, ad, self.seg)
                self.keep.append((x, A, B, ad, y, ws))
                calls.append((x.data_ptr(), x.stride(0), ad.c, y.data_ptr(), y.stride(0),
                              ws.data_ptr(), ws.numel()))
            self.sets.append(calls)
        self.stream = torch.cuda.current_stream().cuda_stream
        self.work = []
        for name in self.names:
            p = projs[name]
            self.work.append(fwd_work(p.h_in, p.h_out, p.ranks, starts, adap))
        self.bytes_per_step = sum(b for b, _ in self.work)
        self.flops_per_step = sum(f for _, f in self.work)

    def step(self, i, events=None):
        lib = self.lib
        k = i % len(self.sets)
        perm_ptr = self.perm.ctypes.data
        if self.request_order and not self.host_rows:
            if self.rows_ev[k] is not None:
                self.rows_ev[k].synchronize()
            perm_ptr = self.rows_host[k].data_ptr()
        st = lib.lora_segments_from_ids(self.ids.ctypes.data, self.T, self.N, perm_ptr,
                                        self.starts.ctypes.data, self.adap.ctypes.data)
        if st:
            raise RuntimeError(lib.lora_last_error().decode())
        calls = self.sets[k]
        segp = ctypes.byref(self.cseg)
        if self.host_rows:
            segp = ctypes.byref(self.cseg_host)
        elif self.request_order:
            import torch
            self.rows_dev[k].copy_(self.rows_host[k], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record()
            self.rows_ev[k] = ev
            segp = ctypes.byref(self.cseg_rows[k])
        for j, (xp, ldx, adc, yp, ldy, wsp, wsb) in enumerate(calls):
            ev = events if events is not None and events[0] == j else None
            if ev is not None:
                ev[1].record()
            st = lib.lora_sgmv_fused(xp, ldx, adc, segp, yp, ldy, None, 0, wsp, wsb, self.stream)
            if ev is not None:
                ev[2].record()
            if st:
                raise RuntimeError(lib.lora_last_error().decode())


EVENT_EVERY = 8  # steps between the steps that carry a pair of timing events (breakdown pass)


def bench_decode(steps, warmup, nsets=16):
    import torch
    from workloads import make_c2_projections
    projs = make_c2_projections(1)
    ds = DecodeStep(projs, nsets)
    for i in range(warmup):
        ds.step(i)
    torch.cuda.synchronize()
    # timed region: wall clock for value, and one pair of HIP events on the
    # launch stream around the whole region for the mean launch duration
    # (GPU time of the region / launches, so inter-launch gaps count against
    # the kernel; no event sits between launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        ds.step(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gpu_per_launch = e0.elapsed_time(e1) * 1e-3 / (3 * steps)
    # breakdown pass (not timed for value): an event pair around one launch
    # of every EVENT_EVERY-th step, the projections in turn; each pair adds a
    # few microseconds of its own
    sampled = list(range(0, steps, EVENT_EVERY))
    ev = {i: (k % 3, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for k, i in enumerate(sampled)}
    for i in range(steps):
        ds.step(warmup + steps + i, ev.get(i))
    torch.cuda.synchronize()
    per_launch = [np.array([a.elapsed_time(b) for (j, a, b) in ev.values() if j == jj]) * 1e-3 for jj in range(3)]
    return ds, (t1 - t0) / steps, gpu_per_launch, per_launch  # seconds


def bench_decode_request_order(steps=200, warmup=20, nsets=16):
    """The decode step with x and y left in request order, the kernels
    gathering x rows and scattering y rows: with the row table as the host
    copy that the launches carry in their arguments (no upload), and with
    the table uploaded to the device every step."""
    import torch
    from workloads import make_c2_projections
    projs = make_c2_projections(1)
    out = []
    for host_rows, name, note in (
            (True, "decode_request_order_token_rows_qwen3_4b_256tok_8x_r32",
             "wall time per step incl. bookkeeping; row table carried in the launch arguments"),
            (False, "decode_request_order_token_rows_uploaded_qwen3_4b_256tok_8x_r32",
             "wall time per step incl. bookkeeping and the row-table upload")):
        ds = DecodeStep(projs, nsets, request_order=True, host_rows=host_rows)
        for i in range(warmup):
            ds.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            ds.step(warmup + i)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        out.append(_entry(name, np.array([sec]), ds.bytes_per_step, ds.flops_per_step, {"note": note}))
        del ds
        torch.cuda.empty_cache()
    return out


def bench_decode_graph(steps=200, warmup=20, nsets=16):
    """The decode step as one replayed HIP graph: the three projections'
    device-planned calls (lora_sgmv_fused_graph: one fused launch each that
    groups the 256 request-order ids itself, every table on the device),
    captured once per rotation set and replayed; wall time and GPU time per
    replay. A second entry captures eight consecutive steps (24 launches)
    per graph, as a serving loop that captures a whole step of many layers
    would: the launches are the same, only the graph boundaries are fewer."""
    import torch
    import lora_adapter_batching_amd as L
    from workloads import make_c2_projections
    projs = make_c2_projections(1)
    p0 = projs["q"]
    T = int(p0.T)
    graphs, keep, set_calls = [], [], []
    work_b = work_f = 0
    perm, starts, adap = L.segments_from_ids(p0.token_ids, p0.N)
    for name in ("q", "o", "gate_up"):
        p = projs[name]
        b, f = fwd_work(p.h_in, p.h_out, p.ranks, starts, adap)
        work_b += b
        work_f += f
    for s in range(nsets):
        calls = []
        for name in ("q", "o", "gate_up"):
            p = projs[name]
            A = [dev_bf16(a) for a in p.A]
            B = [dev_bf16(b) for b in p.B]
            ap = torch.tensor([t.data_ptr() for t in A], dtype=torch.int64, device="cuda")
            bp = torch.tensor([t.data_ptr() for t in B], dtype=torch.int64, device="cuda")
            rk = torch.from_numpy(np.asarray(p.ranks, np.int32).copy()).cuda()
            sc = torch.from_numpy(np.asarray(p.scales, np.float32).copy()).cuda()
            ga = L.GraphAdapters(ap, bp, rk, sc, p.h_in, p.h_out, int(np.max(p.ranks)))
            x = dev_bf16(p.x)
            y = torch.zeros((T, p.h_out), dtype=torch.bfloat16, device="cuda")
            ids = torch.from_numpy(np.asarray(p.token_ids, np.int32).copy()).cuda()
            ws = L.new_workspace_graph(ga, T)
            keep.append((A, B, ap, bp, rk, sc, ga, x, y, ids, ws))
            calls.append((x, ga, ids, y, ws))
        for c in calls:  # warm-up outside the capture
            L.sgmv_fused_graph(*c)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                L.sgmv_fused_graph(*c)
        graphs.append(g)
        set_calls.append(calls)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % nsets].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        graphs[i % nsets].replay()
    e1.record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    gpu = e0.elapsed_time(e1) * 1e-3 / steps
    out = [_entry("decode_step_graph_replay_device_planned_qwen3_4b_256tok_8x_r32", np.array([sec]), work_b, work_f,
                  {"gpu_us_per_step": round(gpu * 1e6, 2),
                   "note": "one HIP graph per step: 3 fused launches that plan on the device, ids on the device"})]
    # eight steps per graph: rotation sets 0-7 and 8-15
    per = 8
    big = []
    for h in range(nsets // per):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for s in range(per * h, per * h + per):
                for c in set_calls[s]:
                    L.sgmv_fused_graph(*c)
        big.append(g)
    torch.cuda.synchronize()
    for i in range(max(2, warmup // per)):
        big[i % len(big)].replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per)
    t0 = time.perf_counter()
    e0.record()
    for i in range(reps):
        big[i % len(big)].replay()
    e1.record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / (reps * per)
    gpu = e0.elapsed_time(e1) * 1e-3 / (reps * per)
    out.append(_entry("decode_step_in_8_step_graph_device_planned_qwen3_4b_256tok_8x_r32", np.array([sec]),
                      work_b, work_f,
                      {"gpu_us_per_step": round(gpu * 1e6, 2),
                       "note": "eight decode steps (24 device-planned launches) per replayed HIP graph"}))
    return out


# ---------------------------------------------------------------------------
# Secondary workloads (HIP events around each call)
# ---------------------------------------------------------------------------
def _upload(prob, L):
    import torch
    if prob.segmented:
        perm = np.arange(prob.T, dtype=np.int32)
        starts = np.concatenate([[0], np.cumsum(prob.seg_lens)]).astype(np.int32)
        adap = np.asarray(prob.seg_adapter, np.int32)
    else:
        perm, starts, adap = L.segments_from_ids(prob.token_ids, prob.N)
    x = dev_bf16(prob.x[perm])
    A = [dev_bf16(a) for a in prob.A]
    B = [dev_bf16(b) for b in prob.B]
    ad = L.Adapters(A, B, prob.ranks, prob.scales, prob.h_in, prob.h_out)
    sg = L.Segments(starts, adap)
    y = torch.zeros((prob.T, prob.h_out), dtype=torch.bfloat16, device="cuda")
    return dict(x=x, A=A, B=B, ad=ad, sg=sg, y=y, starts=starts, adap=adap, perm=perm)


def _time_calls(fn, reps, warm=3):
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    ts = []
    for i in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn(i)
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in ts]) * 1e-3


def _time_region(fn, reps, warm=64):
    """Mean seconds per call of `reps` back-to-back calls between one pair of
    HIP events. For launches shorter than the host's submission time a pair
    of events around each call would time the host, not the kernel. The
    warm-up is long because the first few hundred launches of a fresh process
    can include one multi-millisecond stall of the runtime (seen once, about
    40 ms, between kernels of normal duration in a kernel trace)."""
    import torch
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    b.synchronize()
    return np.array([a.elapsed_time(b) * 1e-3 / reps])


def _entry(name, seconds, bytes_, flops, extra=None):
    seconds = np.asarray(seconds, np.float64)
    med = float(np.median(seconds))
    gbs = bytes_ / med / 1e9
    tfl = flops / med / 1e12
    d = {"workload": name, "us": round(med * 1e6, 2), "GB/s": round(gbs, 1),
         "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "TFLOP/s": round(tfl, 2),
         "mfma_frac": round(tfl / BF16_PEAK_TFLOPS, 5), "bytes": int(bytes_), "flops": int(flops)}
    if seconds.size > 1:  # per-call samples: their spread too
        d["p10_us"] = round(float(np.percentile(seconds, 10)) * 1e6, 2)
        d["p90_us"] = round(float(np.percentile(seconds, 90)) * 1e6, 2)
    if extra:
        d.update(extra)
    return d


def copy_ceiling_gbs(nbytes=1 << 30, reps=10):
    """Achievable HBM rate of a plain device-to-device copy (read + write
    bytes per second), timed with HIP events: the practical ceiling next to
    the 8 TB/s datasheet peak."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    e1.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del a, b
    return 2.0 * nbytes / sec / 1e9


def copy_same_bytes_us(nbytes, nsets=16, reps=200):
    """Mean time of a plain device-to-device copy that moves nbytes in all
    (nbytes / 2 read, nbytes / 2 written), rotating over nsets buffer pairs so
    that the Infinity Cache cannot serve it, launched back to back like the
    decode launches: what a kernel of this size reaches at best."""
    import torch
    half = int(nbytes // 2) // 16 * 16
    src = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    for i in range(nsets):
        dst[i].copy_(src[i])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        dst[i % nsets].copy_(src[i % nsets])
    e1.record()
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del src, dst
    return us


def bench_shrink_expand(reps=20):
    """The separate shrink (x -> u) and expand (u -> y) entry points on the
    prefill batch and on the decode gate_up projection (rotated inputs)."""
    import torch
    import lora_adapter_batching_amd as L
    from workloads import make_c2_projections, make_config
    out = []
    cases = (("prefill_llama3_8b_8192tok_4096x4096_8x_r16", make_config("prefill"), 3),
             ("decode_gate_up_2560x19456_256tok_8x_r32", make_c2_projections(1)["gate_up"], 16))
    for name, prob, nsets in cases:
        sets = [_upload(prob, L) for _ in range(nsets)]
        rmax = int(prob.ranks.max())
        us = [torch.zeros((prob.T, rmax), dtype=torch.float32, device="cuda") for _ in range(nsets)]
        ws = L.new_workspace(L.OP_SHRINK, sets[0]["ad"], sets[0]["sg"])
        st, ad = sets[0]["starts"], sets[0]["adap"]

        def shr(i):
            s = sets[i % nsets]
            L.sgmv_shrink(s["x"], s["ad"], s["sg"], us[i % nsets], ws)

        def exp(i):
            s = sets[i % nsets]
            L.sgmv_expand(us[i % nsets], s["ad"], s["sg"], s["y"], None)
        b, f = shrink_work(prob.h_in, prob.ranks, st, ad)
        out.append(_entry(name + "_shrink", _time_region(shr, 10 * reps), b, f, {"timing": "back-to-back calls"}))
        b, f = expand_work(prob.h_out, prob.ranks, st, ad)
        out.append(_entry(name + "_expand", _time_region(exp, 10 * reps), b, f, {"timing": "back-to-back calls"}))
        del sets, us
        torch.cuda.empty_cache()
    return out


def bench_host(reps=2000):
    """Host-side costs: the token bookkeeping (request-order ids -> segments
    and row table, a counting sort in the library) at decode and
    packed-training sizes, and the host time of one fused decode call
    (validation, planning and the launch itself) through the C ABI."""
    import lora_adapter_batching_amd as L
    lib = L.load()
    out = []
    rng = np.random.default_rng(7)
    for T, N in ((256, 8), (65536, 32)):
        ids = rng.integers(0, N, size=T).astype(np.int32)
        perm = np.zeros(T, np.int32)
        st = np.zeros(N + 2, np.int32)
        ad = np.zeros(N + 1, np.int32)
        n = reps if T <= 4096 else max(20, reps // 50)
        t0 = time.perf_counter()
        for _ in range(n):
            lib.lora_segments_from_ids(ids.ctypes.data, T, N, perm.ctypes.data, st.ctypes.data, ad.ctypes.data)
        us = (time.perf_counter() - t0) / n * 1e6
        out.append({"workload": f"host_bookkeeping_{T}tok_{N}_adapters", "us": round(us, 3),
                    "note": "lora_segments_from_ids through ctypes, host only"})
    return out


def bench_host_call(ds, reps=300):
    """Host time of one fused decode call (q projection) through the C ABI,
    issued while the GPU is kept busy so that launches never wait."""
    import torch
    lib = ds.lib
    xp, ldx, adc, yp, ldy, wsp, wsb = ds.sets[0][0]
    segp = ctypes.byref(ds.cseg)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        lib.lora_sgmv_fused(xp, ldx, adc, segp, yp, ldy, None, 0, wsp, wsb, ds.stream)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    return {"workload": "host_cost_per_fused_decode_call", "us": round((t1 - t0) / reps * 1e6, 2),
            "note": "validation + planning + launch, host side, through ctypes"}


def bench_multi_projection(reps=200, nsets=16):
    """q/k/v-shaped decode over one x (Qwen3-4B-like widths: 2560->4096,
    2560->1024, 2560->1024; 8 adapters of rank 32 per projection; the
    256-token decode batch): one multi-projection launch against one fused
    launch per projection, back-to-back calls on rotated inputs."""
    import torch
    import lora_adapter_batching_amd as L
    from workloads import make_c2_projections, make_custom
    base = make_c2_projections(1)["q"]
    ids = np.asarray(base.token_ids, np.int32)
    perm, starts, adap = L.segments_from_ids(ids, base.N)
    sg = L.Segments(starts, adap)
    outs = (4096, 1024, 1024)
    probs = [make_custom(20 + p, base.h_in, h, list(base.ranks), ids=ids) for p, h in enumerate(outs)]
    sets = []
    for _ in range(nsets):
        x = dev_bf16(base.x[perm])
        ads, ys = [], []
        for pr in probs:
            A = [dev_bf16(a) for a in pr.A]
            B = [dev_bf16(b) for b in pr.B]
            ads.append(L.Adapters(A, B, pr.ranks, pr.scales, pr.h_in, pr.h_out))
            ys.append(torch.zeros((pr.T, pr.h_out), dtype=torch.bfloat16, device="cuda"))
        sets.append((x, ads, ys))
    wsm = L.new_workspace_multi(sets[0][1], sg)
    wss = [L.new_workspace(L.OP_FUSED, a, sg) for a in sets[0][1]]
    # the C arguments of every call are marshalled once, so that the timed
    # loop submits at the library's own host cost (the binding's per-call
    # ctypes arrays would otherwise make this a measurement of Python)
    from lora_adapter_batching_amd import binding as Bd
    lib = L.load()
    stream = torch.cuda.current_stream().cuda_stream
    pre_m, pre_s = [], []
    for x, ads, ys in sets:
        tabs = Bd._multi_tables(ads)
        yp = (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
        ld = (ctypes.c_int64 * len(ys))(*[y.stride(0) for y in ys])
        pre_m.append((tabs, yp, ld, x.data_ptr(), x.stride(0)))
        pre_s.append([(x.data_ptr(), x.stride(0), a.c, y.data_ptr(), y.stride(0), w.data_ptr(), w.numel())
                      for a, y, w in zip(ads, ys, wss)])
    segp = sg.c
    wsm_p, wsm_n = wsm.data_ptr(), wsm.numel()

    def multi(i):
        tabs, yp, ld, xp, ldx = pre_m[i % nsets]
        st = lib.lora_sgmv_fused_multi(xp, ldx, len(probs), ctypes.cast(tabs, ctypes.c_void_p), segp,
                                       ctypes.cast(yp, ctypes.c_void_p), ctypes.cast(ld, ctypes.c_void_p),
                                       wsm_p, wsm_n, stream)
        if st:
            raise RuntimeError(lib.lora_last_error().decode())

    def single(i):
        for xp, ldx, ac, yp, ldy, wp, wn in pre_s[i % nsets]:
            st = lib.lora_sgmv_fused(xp, ldx, ac, segp, yp, ldy, None, 0, wp, wn, stream)
            if st:
                raise RuntimeError(lib.lora_last_error().decode())
    tm = float(_time_region(multi, reps)[0])
    ts = float(_time_region(single, reps)[0])
    # algorithmic bytes: each projection's, with x counted once (it is shared)
    n_active = len(active_token_ranks(probs[0].ranks, starts, adap))
    b = sum(fwd_work(pr.h_in, pr.h_out, pr.ranks, starts, adap)[0] for pr in probs)
    b -= (len(probs) - 1) * 2 * n_active * base.h_in
    f = sum(fwd_work(pr.h_in, pr.h_out, pr.ranks, starts, adap)[1] for pr in probs)
    return [_entry("decode_qkv_multi_projection_one_launch_256tok_8x_r32", np.array([tm]), b, f,
                   {"timing": "back-to-back calls", "three_launches_us": round(ts * 1e6, 2),
                    "speedup_vs_three_launches": round(ts / tm, 3)})]


def bench_secondary(reps=20):
    import torch
    import lora_adapter_batching_amd as L
    from workloads import make_config
    out = bench_decode_request_order() + bench_decode_graph()
    torch.cuda.empty_cache()
    out += bench_multi_projection()
    torch.cuda.empty_cache()
    out += bench_shrink_expand(reps)
    torch.cuda.empty_cache()
    for cfg, nsets in (("prefill", 3), ("hetero", 2)):
        prob = make_config(cfg)
        sets = [_upload(prob, L) for _ in range(nsets)]
        ws = L.new_workspace(L.OP_FUSED, sets[0]["ad"], sets[0]["sg"])
        b, f = fwd_work(prob.h_in, prob.h_out, prob.ranks, sets[0]["starts"], sets[0]["adap"])

        def fn(i, sets=sets, ws=ws):
            s = sets[i % len(sets)]
            L.sgmv_fused(s["x"], s["ad"], s["sg"], s["y"], None, ws)
        sec = _time_calls(fn, reps)
        name = {"prefill": "prefill_llama3_8b_8192tok_4096x4096_8x_r16",
                "hetero": "hetero_mlp_up_4096tok_4096x14336_32x_r8-128"}[cfg]
        out.append(_entry(name, sec, b, f))
        del sets
        torch.cuda.empty_cache()
    # packed training: fused forward (saving u) + packed backward
    prob = make_config("train")
    s = _upload(prob, L)
    dy = dev_bf16(prob.dy)
    rmax = int(prob.ranks.max())
    u = torch.zeros((prob.T, rmax), dtype=torch.float32, device="cuda")
    dx = torch.zeros((prob.T, prob.h_in), dtype=torch.bfloat16, device="cuda")
    dA = [torch.zeros((int(r), prob.h_in), dtype=torch.float32, device="cuda") for r in prob.ranks]
    dB = [torch.zeros((prob.h_out, int(r)), dtype=torch.float32, device="cuda") for r in prob.ranks]
    pa = torch.tensor([t.data_ptr() for t in dA], dtype=torch.int64, device="cuda")
    pb = torch.tensor([t.data_ptr() for t in dB], dtype=torch.int64, device="cuda")
    wsf = L.new_workspace(L.OP_FUSED, s["ad"], s["sg"])
    wsb = L.new_workspace(L.OP_BACKWARD, s["ad"], s["sg"])
    bf, ff = fwd_work(prob.h_in, prob.h_out, prob.ranks, s["starts"], s["adap"], save_u=True)
    bb, fb = bwd_work(prob.h_in, prob.h_out, prob.ranks, s["starts"], s["adap"])
    sf = _time_calls(lambda i: L.sgmv_fused(s["x"], s["ad"], s["sg"], s["y"], u, wsf), reps // 2)
    sb = _time_calls(lambda i: L.packed_backward(s["x"], dy, u, s["ad"], s["sg"], dx, pa, pb, 0, wsb),
                     reps // 2)
    out.append(_entry("train_fwd_qwen2p5_7b_65536tok_3584x3584_32x_r8-64", sf, bf, ff))
    out.append(_entry("train_bwd_qwen2p5_7b_65536tok_3584x3584_32x_r8-64", sb, bb, fb))
    out.append(_entry("train_fwd_bwd_qwen2p5_7b", np.array([np.median(sf) + np.median(sb)]), bf + bb,
                      ff + fb))
    return out


# ---------------------------------------------------------------------------
# Packed vs one-adapter-at-a-time: N adapters in one call against N calls of
# one adapter each, on the same kernels and the same tokens
# ---------------------------------------------------------------------------
def _adapter_subset(L, A, B, ranks, scales, h_in, h_out, idx):
    return L.Adapters([A[i] for i in idx], [B[i] for i in idx], np.asarray(ranks)[idx],
                      np.asarray(scales)[idx], h_in, h_out)


def _sweep_decode(L, counts, reps):
    """gate_up (2560->19456, rank 32) over the 256-token decode batch: token
    ids uniform in [0, 8) are folded onto n adapters (id mod n)."""
    import torch
    from workloads import make_c2_projections
    p = make_c2_projections(1)["gate_up"]
    A = [dev_bf16(a) for a in p.A]
    B = [dev_bf16(b) for b in p.B]
    out = []
    for n in counts:
        ids = (np.asarray(p.token_ids) % n).astype(np.int32)
        perm, starts, adap = L.segments_from_ids(ids, n)
        x = dev_bf16(p.x[perm])
        y = torch.zeros((p.T, p.h_out), dtype=torch.bfloat16, device="cuda")
        ad = _adapter_subset(L, A, B, p.ranks, p.scales, p.h_in, p.h_out, list(range(n)))
        sg = L.Segments(starts, adap)
        ws = L.new_workspace(L.OP_FUSED, ad, sg)
        packed = _time_calls(lambda i: L.sgmv_fused(x, ad, sg, y, None, ws), reps)
        # one adapter per call: its rows only (views of the same buffers)
        single = []
        for a in range(n):
            t0, t1 = int(starts[a]), int(starts[a + 1])
            if t1 == t0:
                continue
            ad1 = _adapter_subset(L, A, B, p.ranks, p.scales, p.h_in, p.h_out, [a])
            sg1 = L.Segments(np.array([0, t1 - t0], np.int32), np.array([0], np.int32))
            single.append((x[t0:t1], ad1, sg1, y[t0:t1], L.new_workspace(L.OP_FUSED, ad1, sg1)))

        def seq(i):
            for xs, a1, s1, ys, w1 in single:
                L.sgmv_fused(xs, a1, s1, ys, None, w1)
        sequential = _time_calls(seq, reps)
        b, _ = fwd_work(p.h_in, p.h_out, p.ranks[:n], starts, adap)
        tp, tsq = float(np.median(packed)), float(np.median(sequential))
        out.append({"adapters": n, "tokens": int(p.T), "packed_us": round(tp * 1e6, 2),
                    "sequential_us": round(tsq * 1e6, 2), "speedup": round(tsq / tp, 3),
                    "packed_GBs": round(b / tp / 1e9, 1), "launches_sequential": len(single)})
        log(f"sweep decode n={n}: {out[-1]}")
    return out


def _sweep_train(L, counts, reps):
    """Packed training (3584->3584, ranks in {8,16,32,64}, 4 x 512 tokens per
    adapter, adapter-major): fused forward saving u, then the packed
    backward, for the first n adapters in one call each, against the same two
    calls made once per adapter."""
    import torch
    from workloads import make_config
    prob = make_config("train")
    per = int(prob.T // prob.N)  # tokens per adapter
    x_all = dev_bf16(prob.x)
    dy_all = dev_bf16(prob.dy)
    A = [dev_bf16(a) for a in prob.A]
    B = [dev_bf16(b) for b in prob.B]
    rmax = int(prob.ranks.max())
    dA = [torch.zeros((int(r), prob.h_in), dtype=torch.float32, device="cuda") for r in prob.ranks]
    dB = [torch.zeros((prob.h_out, int(r)), dtype=torch.float32, device="cuda") for r in prob.ranks]
    seg_lens = np.asarray(prob.seg_lens)
    seg_ad = np.asarray(prob.seg_adapter)
    out = []

    def case(idx):
        """Buffers for one call over adapters idx (their tokens are contiguous)."""
        t0, t1 = idx[0] * per, (idx[-1] + 1) * per
        sel = np.isin(seg_ad, idx)
        lens = seg_lens[sel]
        local = np.searchsorted(np.asarray(idx), seg_ad[sel]).astype(np.int32)
        starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        ad = _adapter_subset(L, A, B, prob.ranks, prob.scales, prob.h_in, prob.h_out, list(idx))
        sg = L.Segments(starts, local)
        x, dy = x_all[t0:t1], dy_all[t0:t1]
        y = torch.zeros((t1 - t0, prob.h_out), dtype=torch.bfloat16, device="cuda")
        dx = torch.zeros((t1 - t0, prob.h_in), dtype=torch.bfloat16, device="cuda")
        u = torch.zeros((t1 - t0, rmax), dtype=torch.float32, device="cuda")
        pa = torch.tensor([dA[i].data_ptr() for i in idx], dtype=torch.int64, device="cuda")
        pb = torch.tensor([dB[i].data_ptr() for i in idx], dtype=torch.int64, device="cuda")
        wsf = L.new_workspace(L.OP_FUSED, ad, sg)
        wsb = L.new_workspace(L.OP_BACKWARD, ad, sg)

        def run():
            L.sgmv_fused(x, ad, sg, y, u, wsf)
            L.packed_backward(x, dy, u, ad, sg, dx, pa, pb, 0, wsb)
        return run, starts, local

    for n in counts:
        run_p, starts, local = case(list(range(n)))
        packed = _time_calls(lambda i: run_p(), reps)
        singles = [case([a])[0] for a in range(n)]

        def seq(i):
            for r in singles:
                r()
        sequential = _time_calls(seq, reps)
        bf, ff = fwd_work(prob.h_in, prob.h_out, prob.ranks[:n], starts, local, save_u=True)
        bb, fb = bwd_work(prob.h_in, prob.h_out, prob.ranks[:n], starts, local)
        tp, tsq = float(np.median(packed)), float(np.median(sequential))
        out.append({"adapters": n, "tokens": n * per, "packed_us": round(tp * 1e6, 1),
                    "sequential_us": round(tsq * 1e6, 1), "speedup": round(tsq / tp, 3),
                    "packed_tokens_per_s": round(n * per / tp), "packed_GBs": round((bf + bb) / tp / 1e9, 1),
                    "packed_TFLOPs": round((ff + fb) / tp / 1e12, 2)})
        log(f"sweep train n={n}: {out[-1]}")
        del singles, run_p
        torch.cuda.empty_cache()
    return out


def bench_adapter_sweep(reps=20):
    import lora_adapter_batching_amd as L
    L.load()
    return {"sweep": "packed_vs_sequential_adapters",
            "decode_gate_up_2560x19456_256tok_r32": _sweep_decode(L, (1, 2, 4, 8), reps),
            "train_fwd_bwd_3584x3584_2048tok_per_adapter": _sweep_train(L, (1, 2, 4, 8, 16, 32), reps // 2)}


def bench_only(name, reps=5):
    """One secondary workload alone (for counter runs): 'prefill' and
    'hetero' run the fused forward, 'train' the fused forward saving u and
    then the packed backward, each `reps` times on rotated inputs."""
    import torch
    import lora_adapter_batching_amd as L
    from workloads import make_config
    prob = make_config(name)
    nsets = 1 if name == "train" else 2
    sets = [_upload(prob, L) for _ in range(nsets)]
    s0 = sets[0]
    out = {"only": name, "reps": reps}
    if name != "train":
        ws = L.new_workspace(L.OP_FUSED, s0["ad"], s0["sg"])
        sec = _time_calls(lambda i: L.sgmv_fused(sets[i % nsets]["x"], sets[i % nsets]["ad"], sets[i % nsets]["sg"],
                                                 sets[i % nsets]["y"], None, ws), reps, warm=1)
        b, f = fwd_work(prob.h_in, prob.h_out, prob.ranks, s0["starts"], s0["adap"])
        out["fwd"] = _entry(name, sec, b, f)
    else:
        dy = dev_bf16(prob.dy)
        u = torch.zeros((prob.T, int(prob.ranks.max())), dtype=torch.float32, device="cuda")
        dx = torch.zeros((prob.T, prob.h_in), dtype=torch.bfloat16, device="cuda")
        dA = [torch.zeros((int(r), prob.h_in), dtype=torch.float32, device="cuda") for r in prob.ranks]
        dB = [torch.zeros((prob.h_out, int(r)), dtype=torch.float32, device="cuda") for r in prob.ranks]
        pa = torch.tensor([t.data_ptr() for t in dA], dtype=torch.int64, device="cuda")
        pb = torch.tensor([t.data_ptr() for t in dB], dtype=torch.int64, device="cuda")
        wsf = L.new_workspace(L.OP_FUSED, s0["ad"], s0["sg"])
        wsb = L.new_workspace(L.OP_BACKWARD, s0["ad"], s0["sg"])
        sf = _time_calls(lambda i: L.sgmv_fused(s0["x"], s0["ad"], s0["sg"], s0["y"], u, wsf), reps, warm=1)
        sb = _time_calls(lambda i: L.packed_backward(s0["x"], dy, u, s0["ad"], s0["sg"], dx, pa, pb, 0, wsb),
                         reps, warm=1)
        bf, ff = fwd_work(prob.h_in, prob.h_out, prob.ranks, s0["starts"], s0["adap"], save_u=True)
        bb, fb = bwd_work(prob.h_in, prob.h_out, prob.ranks, s0["starts"], s0["adap"])
        out["fwd"] = _entry(name + "_fwd", sf, bf, ff)
        out["bwd"] = _entry(name + "_bwd", sb, bb, fb)
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on the host cores
# ---------------------------------------------------------------------------
def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, min_s=0.3, max_reps=20):
    """Seconds per call of fn (repeated until min_s has passed, at least once)."""
    n, t0 = 0, time.perf_counter()
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if dt >= min_s or n >= max_reps:
            return dt / n


def bench_cpu(bytes_per_step, budget_s=6.0):
    """The fp64 oracle timed on the host cores: the headline decode step (the
    value, in the metric's unit), then every workload once per thread count
    (all cores, and one thread for the forward workloads) with its tokens/s
    and GFLOP/s of algorithmic work."""
    from oracle import oracle
    from workloads import make_c2_projections, make_config
    threads_all = oracle.num_threads()
    projs = make_c2_projections(1)
    batches = {k: oracle.Batch(p) for k, p in projs.items()}

    def decode_step():
        for k in ("q", "o", "gate_up"):
            p = projs[k]
            oracle.segments_from_ids(p.token_ids, p.N)
            batches[k].forward()

    n = 0
    t0 = time.perf_counter()
    while True:
        decode_step()
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / n
    per_config = []

    def record(name, fn, tokens, bytes_, flops, threads):
        oracle.set_num_threads(threads)
        sec = _timed(fn)
        per_config.append({"workload": name, "threads": threads, "seconds": round(sec, 5),
                           "tokens_per_s": round(tokens / sec, 1), "GFLOP/s": round(flops / sec / 1e9, 3),
                           "GB/s": round(bytes_ / sec / 1e9, 4)})
        log(f"cpu {name} threads={threads}: {sec * 1e3:.2f} ms")

    d_b = d_f = 0
    perm, st, ad = oracle.segments_from_ids(projs["q"].token_ids, projs["q"].N)
    for k in ("q", "o", "gate_up"):
        p = projs[k]
        b, f = fwd_work(p.h_in, p.h_out, p.ranks, st, ad)
        d_b += b
        d_f += f
    fwd_cases = []
    tiny = make_config("tiny")
    tb = oracle.Batch(tiny)
    tperm, tst, tad = oracle.segments_from_ids(tiny.token_ids, tiny.N)
    fwd_cases.append(("tiny_16tok_256x256_4x_r8", lambda: (oracle.segments_from_ids(tiny.token_ids, tiny.N),
                                                           tb.forward()), tiny.T,
                      *fwd_work(tiny.h_in, tiny.h_out, tiny.ranks, tst, tad)))
    fwd_cases.append(("decode_step_qwen3_4b_256tok_8x_r32", decode_step, 256, d_b, d_f))
    for name, cfg in (("prefill_llama3_8b_8192tok_4096x4096_8x_r16", "prefill"),
                      ("hetero_mlp_up_4096tok_4096x14336_32x_r8-128", "hetero")):
        prob = make_config(cfg)
        bt = oracle.Batch(prob)
        b, f = fwd_work(prob.h_in, prob.h_out, prob.ranks, bt.seg_starts, bt.seg_adapter)
        fwd_cases.append((name, bt.forward, prob.T, b, f))
    for name, fn, tok, b, f in fwd_cases:
        for th in (threads_all, 1):
            record(name, fn, tok, b, f, th)
    del fwd_cases
    train = make_config("train")
    trb = oracle.Batch(train)
    del train.x, train.dy
    bf, ff = fwd_work(trb.prob.h_in, trb.prob.h_out, trb.ranks, trb.seg_starts, trb.seg_adapter, save_u=True)
    bb, fb = bwd_work(trb.prob.h_in, trb.prob.h_out, trb.ranks, trb.seg_starts, trb.seg_adapter)

    def train_step():
        _, u = trb.forward()
        trb.backward(u)

    record("train_fwd_bwd_qwen2p5_7b_65536tok_3584x3584_32x_r8-64", train_step, trb.prob.T, bf + bb, ff + fb,
           threads_all)
    oracle.set_num_threads(threads_all)
    return {"value": round(bytes_per_step / dt / 1e9, 4), "unit": "GB/s", "cores": threads_all,
            "kind": "oracle", "cpu_model": _cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{n} full decode steps (grouping + q, o, gate_up forward, 256 tokens) in fp64, "
                      f"{dt * 1e3:.1f} ms per step",
            "per_config": per_config}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", choices=["prefill", "hetero", "train"],
                    help="run one secondary workload alone (counter runs)")
    ap.add_argument("--reps", type=int, default=5, help="repetitions for --only")
    ap.add_argument("--sweep-adapters", action="store_true",
                    help="only time N packed adapters in one call against N one-adapter calls")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel()}))
        return
    if args.only:
        print(json.dumps(bench_only(args.only, args.reps)), flush=True)
        return
    if args.sweep_adapters:
        print(json.dumps(bench_adapter_sweep()), flush=True)
        return
    import lora_adapter_batching_amd as L
    L.load()
    log("decode step")
    ds, sec_per_step, avg_launch, per_launch = bench_decode(args.steps, args.warmup)
    value = ds.bytes_per_step / sec_per_step / 1e9
    # dominant kernel: the fused launch (sgmv_fwd_kernel), 3 launches per step
    bytes_per_launch = ds.bytes_per_step / 3.0
    achieved = bytes_per_launch / avg_launch / 1e9
    traffic = load_traffic(WORKLOAD)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": KERNEL, "avg_launch_us": round(avg_launch * 1e6, 3),
            "launch_us_event_pairs": {n: round(float(np.median(per_launch[j])) * 1e6, 3)
                                      for j, n in enumerate(ds.names)},
            "algorithmic_bytes_per_launch": round(bytes_per_launch),
            "event_every_steps": EVENT_EVERY}
    gate = ds.work[2][0] / float(np.median(per_launch[2])) / 1e9
    roof["gate_up_GBs_event_pair"] = round(gate, 1)
    roof["copy_ceiling_GBs"] = round(copy_ceiling_gbs(), 1)
    # the same bytes as one launch, moved by a plain copy (launch-latency floor)
    roof["copy_same_bytes_us"] = {n: round(copy_same_bytes_us(ds.work[j][0]), 2) for j, n in enumerate(ds.names)}
    out = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec_per_step * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": WORKLOAD, "tokens": ds.T, "adapters": ds.N, "rank": 32,
                      "projections": {"q": [2560, 2560], "o": [2560, 2560], "gate_up": [2560, 19456]},
                      "bytes_per_step": int(ds.bytes_per_step), "flops_per_step": int(ds.flops_per_step),
                      "rotation_sets": len(ds.sets)},
           "roofline": roof}
    if not args.no_secondary:
        # (extra launches: kept out of --no-secondary runs, whose launch
        # sequence the profile summaries split into q, o, gate_up)
        host = bench_host() + [bench_host_call(ds)]
        log("secondary workloads")
        del ds
        torch.cuda.empty_cache()
        out["secondary"] = host + bench_secondary()
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = bench_cpu(out["config"]["bytes_per_step"])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
