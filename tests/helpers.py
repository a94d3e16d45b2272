"""Shared test helpers: move seeded workloads to the GPU, run the library,
and compare with the fp64 oracle.

Tolerances. bf16 outputs (y, dx): max|gpu - oracle| / max|oracle| <= 1e-2 per
tensor (the parity bar for bf16 inputs with fp32 accumulation). fp32 outputs
(u, dA_i, dB_i): 1e-3 -- inputs are exact bf16, sums are fp32 and every fp32
operand of a bf16 MFMA is split into a bf16 hi + lo pair (about 16 mantissa
bits), so the expected error is ~1e-5; 1e-3 leaves a wide margin while still
catching a dropped lo part or a wrong scale.
"""
from __future__ import annotations

import numpy as np

from oracle import oracle

BF16_TOL = 1e-2
FP32_TOL = 1e-3


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def dev_bf16(bits: np.ndarray):
    import torch
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to("cuda")


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class GpuProblem:
    """A workload uploaded to the GPU and grouped by the library's bookkeeping.

    use_token_rows: keep x/y/dy in request order on the device and pass the
    permutation as token_rows (in-kernel gather/scatter); otherwise rows are
    permuted on the host before upload. host_rows ("only" or "both") also
    passes the permutation as the host copy token_rows_host, alone or beside
    the device table.
    """

    def __init__(self, prob, use_token_rows: bool = False, y0: bool = False, host_tables: bool = True,
                 host_rows: str = ""):
        import torch
        import lora_adapter_batching_amd as L
        self.prob = prob
        if prob.segmented:
            self.perm = np.arange(prob.T, dtype=np.int32)
            self.seg_starts = np.concatenate([[0], np.cumsum(prob.seg_lens)]).astype(np.int32)
            self.seg_adapter = np.asarray(prob.seg_adapter, np.int32)
        else:
            self.perm, self.seg_starts, self.seg_adapter = L.segments_from_ids(prob.token_ids, prob.N)
        self.use_token_rows = use_token_rows
        order = np.arange(prob.T) if use_token_rows else self.perm
        self.x = dev_bf16(prob.x[order]) if prob.T else torch.zeros((0, prob.h_in), dtype=torch.bfloat16, device="cuda")
        self.dy = dev_bf16(prob.dy[order]) if prob.dy is not None else None
        if prob.y0 is not None:
            self.y_init = dev_bf16(prob.y0[order])
        else:
            self.y_init = torch.zeros((prob.T, prob.h_out), dtype=torch.bfloat16, device="cuda")
        self.A = [dev_bf16(a) if a.size else None for a in prob.A]
        self.B = [dev_bf16(b) if b.size else None for b in prob.B]
        self.adapters = L.Adapters(self.A, self.B, prob.ranks, prob.scales, prob.h_in, prob.h_out,
                                   host_tables=host_tables)
        tr = torch.from_numpy(self.perm.copy()).to("cuda") if use_token_rows else None
        # host_rows: "" (device table only), "only" (host copy alone), "both"
        rows_host = self.perm.copy() if use_token_rows and host_rows else None
        if use_token_rows and host_rows == "only":
            tr = None
        self.token_rows = tr
        self.segments = L.Segments(self.seg_starts, self.seg_adapter, tr, rows_host)
        self.rmax = max(1, int(np.max(prob.ranks)) if prob.N else 1)

    def sorted_rows(self, t) -> np.ndarray:
        """Device rows -> host fp64 array in sorted-position order."""
        a = to_f64(t)
        return a[self.perm] if self.use_token_rows else a

    def new_y(self):
        return self.y_init.clone()

    def new_u(self, fill=float("nan")):
        import torch
        return torch.full((self.prob.T, self.rmax), fill, dtype=torch.float32, device="cuda")


def oracle_batch(prob) -> "oracle.Batch":
    return oracle.Batch(prob)
