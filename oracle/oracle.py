"""Python side of the fp64 CPU oracle (ctypes over lora_oracle.c).

TEST INFRASTRUCTURE ONLY: the slow, obviously correct reference for the HIP
library. Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module. It imports nothing from the library package;
the two share only the seeded input generators in ``workloads``.

Every bf16 input is widened exactly to fp64 here (a bf16 bit pattern shifted
into the high half of a float32 word); all arithmetic then happens in the C
file in fp64. What the functions compute is stated in lora_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lora_oracle.c")
_LIB = os.path.join(_HERE, "liblora_oracle.so")
_lib = None

_I32P = ctypes.POINTER(ctypes.c_int32)
_F64P = ctypes.POINTER(ctypes.c_double)
_F64PP = ctypes.POINTER(_F64P)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, no FMA contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        lib.oracle_segments_from_ids.restype = ctypes.c_int
        lib.oracle_segments_from_ids.argtypes = [_I32P, ctypes.c_int32, ctypes.c_int32, _I32P,
                                                 _I32P, _I32P]
        lib.oracle_forward.restype = None
        lib.oracle_forward.argtypes = [ctypes.c_int32] * 4 + [_I32P, _I32P, _I32P, _F64P, _F64PP,
                                                              _F64PP, _F64P, _F64P, _F64P,
                                                              ctypes.c_int32]
        lib.oracle_backward.restype = None
        lib.oracle_backward.argtypes = ([ctypes.c_int32] * 4 +
                                        [_I32P, _I32P, _I32P, _F64P, _F64PP, _F64PP,
                                         ctypes.c_int32, _F64P, _F64P, _F64P, _F64P,
                                         ctypes.c_int32, _F64P, _F64PP, _F64PP, ctypes.c_int32])
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def widen(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _ptr_table(mats: Sequence[Optional[np.ndarray]]):
    arr = (_F64P * max(1, len(mats)))()
    for i, m in enumerate(mats):
        arr[i] = _p(m, _F64P) if m is not None and m.size > 0 else _F64P()
    return arr


def segments_from_ids(ids: np.ndarray, N: int):
    """(perm, seg_starts[N+2], seg_adapter[N+1]); raises on an id outside [-1, N)."""
    ids = _i32(ids)
    T = ids.shape[0]
    perm = np.zeros(max(T, 1), np.int32)
    starts = np.zeros(N + 2, np.int32)
    adap = np.zeros(N + 1, np.int32)
    rc = _load().oracle_segments_from_ids(_p(ids, _I32P), T, N, _p(perm, _I32P),
                                          _p(starts, _I32P), _p(adap, _I32P))
    if rc != 0:
        raise ValueError("adapter id outside [-1, N)")
    return perm[:T], starts, adap


def forward(x: np.ndarray, A: List[np.ndarray], B: List[np.ndarray], ranks, scales,
            seg_starts, seg_adapter, y0: Optional[np.ndarray] = None, h_out: Optional[int] = None):
    """fp64 forward. x [T, h_in] float64; A[i] [r_i, h_in], B[i] [h_out, r_i]
    float64. Returns (y [T, h_out], u [T, max(r)]); rows of u for skipped
    tokens are NaN (never written)."""
    x = np.ascontiguousarray(x, np.float64)
    T, h_in = x.shape
    ranks = _i32(ranks)
    if h_out is None:
        h_out = next(b.shape[0] for b in B)
    scales = np.ascontiguousarray(scales, np.float64)
    seg_starts, seg_adapter = _i32(seg_starts), _i32(seg_adapter)
    S = seg_adapter.shape[0]
    assert seg_starts.shape[0] == S + 1 and int(seg_starts[-1]) == T
    ldu = max(1, int(ranks.max()) if ranks.size else 1)
    y = (np.zeros((T, h_out)) if y0 is None else np.array(y0, dtype=np.float64, copy=True))
    y = np.ascontiguousarray(y)
    u = np.full((T, ldu), np.nan)
    Ac = [np.ascontiguousarray(a, np.float64) for a in A]
    Bc = [np.ascontiguousarray(b, np.float64) for b in B]
    _load().oracle_forward(T, h_in, h_out, S, _p(seg_starts, _I32P), _p(seg_adapter, _I32P),
                           _p(ranks, _I32P), _p(scales, _F64P), _ptr_table(Ac), _ptr_table(Bc),
                           _p(x, _F64P), _p(y, _F64P), _p(u, _F64P), ldu)
    return y, u


def backward(x, dy, u, A, B, ranks, scales, seg_starts, seg_adapter, dx0=None, want_dx=True,
             dA0=None, dB0=None, accumulate=False):
    """fp64 backward given the forward's u. Returns (du, dx, dA list, dB list).
    Rows of du for skipped tokens are NaN; dx is None if want_dx is False."""
    x = np.ascontiguousarray(x, np.float64)
    dy = np.ascontiguousarray(dy, np.float64)
    T, h_in = x.shape
    h_out = dy.shape[1]
    ranks = _i32(ranks)
    N = ranks.shape[0]
    scales = np.ascontiguousarray(scales, np.float64)
    seg_starts, seg_adapter = _i32(seg_starts), _i32(seg_adapter)
    S = seg_adapter.shape[0]
    ldu = u.shape[1]
    u = np.ascontiguousarray(np.nan_to_num(u, nan=0.0), np.float64)
    du = np.full((T, ldu), np.nan)
    dx = None
    if want_dx:
        dx = np.zeros((T, h_in)) if dx0 is None else np.array(dx0, dtype=np.float64, copy=True)
        dx = np.ascontiguousarray(dx)
    dA = [np.zeros((int(r), h_in)) if (dA0 is None) else np.array(dA0[i], dtype=np.float64)
          for i, r in enumerate(ranks)]
    dB = [np.zeros((h_out, int(r))) if (dB0 is None) else np.array(dB0[i], dtype=np.float64)
          for i, r in enumerate(ranks)]
    Ac = [np.ascontiguousarray(a, np.float64) for a in A]
    Bc = [np.ascontiguousarray(b, np.float64) for b in B]
    _load().oracle_backward(T, h_in, h_out, S, _p(seg_starts, _I32P), _p(seg_adapter, _I32P),
                            _p(ranks, _I32P), _p(scales, _F64P), _ptr_table(Ac), _ptr_table(Bc),
                            N, _p(x, _F64P), _p(dy, _F64P), _p(u, _F64P), _p(du, _F64P), ldu,
                            _p(dx, _F64P) if dx is not None else _F64P(), _ptr_table(dA),
                            _ptr_table(dB), 1 if accumulate else 0)
    return du, dx, dA, dB


# ---------------------------------------------------------------------------
# Problem-level helpers (inputs from workloads.Problem)
# ---------------------------------------------------------------------------
class Batch:
    """A workload grouped into segments by the oracle's own bookkeeping.

    For request-order workloads the tokens are grouped by
    segments_from_ids; `perm[p]` is the request index of sorted position p and
    x/dy/y0 are gathered accordingly. Segment-based workloads are used as
    given. All float arrays are fp64 widenings of the bf16 inputs.
    """

    def __init__(self, prob):
        self.prob = prob
        if prob.segmented:
            self.perm = np.arange(prob.T, dtype=np.int32)
            self.seg_starts = np.concatenate([[0], np.cumsum(prob.seg_lens)]).astype(np.int32)
            self.seg_adapter = np.asarray(prob.seg_adapter, np.int32)
        else:
            self.perm, self.seg_starts, self.seg_adapter = segments_from_ids(prob.token_ids, prob.N)
        self.x = widen(prob.x)[self.perm]
        self.A = [widen(a) for a in prob.A]
        self.B = [widen(b) for b in prob.B]
        self.dy = widen(prob.dy)[self.perm] if prob.dy is not None else None
        self.y0 = widen(prob.y0)[self.perm] if prob.y0 is not None else None
        self.ranks = np.asarray(prob.ranks, np.int32)
        self.scales = np.asarray(prob.scales, np.float64)

    def token_adapter(self) -> np.ndarray:
        a = np.full(self.prob.T, -1, np.int32)
        for g in range(len(self.seg_adapter)):
            a[self.seg_starts[g]:self.seg_starts[g + 1]] = self.seg_adapter[g]
        return a

    def forward(self):
        return forward(self.x, self.A, self.B, self.ranks, self.scales, self.seg_starts,
                       self.seg_adapter, self.y0, self.prob.h_out)

    def forward_tokens(self, rows: np.ndarray):
        """Forward for a subset of sorted positions only (each token is
        independent): returns (y rows, u rows)."""
        rows = np.asarray(rows, np.int64)
        a = self.token_adapter()[rows]
        starts = np.arange(len(rows) + 1, dtype=np.int32)
        y0 = self.y0[rows] if self.y0 is not None else None
        return forward(self.x[rows], self.A, self.B, self.ranks, self.scales, starts, a, y0,
                       self.prob.h_out)

    def backward(self, u=None, want_dx=True, dx0=None):
        if u is None:
            _, u = self.forward()
        return backward(self.x, self.dy, u, self.A, self.B, self.ranks, self.scales,
                        self.seg_starts, self.seg_adapter, dx0=dx0, want_dx=want_dx)

    def backward_adapters(self, adapters: Sequence[int], want_dx=True):
        """Backward restricted to every token of the given adapters (their
        dA/dB reductions are complete). Returns (rows, du, dx, dA, dB) where
        rows are the sorted positions involved."""
        a = self.token_adapter()
        keep = np.isin(a, np.asarray(adapters))
        rows = np.nonzero(keep)[0]
        sub_a = a[rows]
        starts = np.arange(len(rows) + 1, dtype=np.int32)
        x = self.x[rows]
        _, u = forward(x, self.A, self.B, self.ranks, self.scales, starts, sub_a, None,
                       self.prob.h_out)
        du, dx, dA, dB = backward(x, self.dy[rows], u, self.A, self.B, self.ranks, self.scales,
                                  starts, sub_a, want_dx=want_dx)
        return rows, du, dx, dA, dB
