"""ctypes binding of liblora_sgmv.so (argument marshalling only).

Every computation runs in the HIP library; this module only turns torch
tensors and numpy arrays into the pointers and sizes of the C ABI declared
in include/lora_sgmv.h, and raises LoraError on a non-zero status. There is
no fallback path: if the library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblora_sgmv.so")

LORA_OK = 0
LORA_INVALID_ARGUMENT = 1
LORA_UNSUPPORTED = 2
LORA_WORKSPACE_TOO_SMALL = 3
LORA_DEVICE_ERROR = 4

OP_SHRINK, OP_EXPAND, OP_FUSED, OP_BACKWARD = 0, 1, 2, 3
GRAD_ACCUMULATE = 1


class LoraError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class CAdapters(ctypes.Structure):
    _fields_ = [("num_adapters", ctypes.c_int32), ("h_in", ctypes.c_int32),
                ("h_out", ctypes.c_int32), ("A_ptrs", ctypes.c_void_p),
                ("B_ptrs", ctypes.c_void_p), ("ranks", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("A_ptrs_host", ctypes.c_void_p),
                ("B_ptrs_host", ctypes.c_void_p)]


class CSegments(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_segments", ctypes.c_int32),
                ("seg_starts", ctypes.c_void_p), ("seg_adapter", ctypes.c_void_p),
                ("token_rows", ctypes.c_void_p), ("token_rows_host", ctypes.c_void_p)]


class CGraphAdapters(ctypes.Structure):
    _fields_ = [("num_adapters", ctypes.c_int32), ("h_in", ctypes.c_int32), ("h_out", ctypes.c_int32),
                ("max_rank", ctypes.c_int32), ("A_ptrs", ctypes.c_void_p), ("B_ptrs", ctypes.c_void_p),
                ("ranks", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


EXPORTS = ["lora_segments_from_ids", "lora_workspace_size", "lora_sgmv_shrink", "lora_sgmv_expand",
           "lora_sgmv_fused", "lora_packed_backward", "lora_workspace_size_multi",
           "lora_sgmv_fused_multi", "lora_sgmv_fused_noalloc", "lora_workspace_size_graph",
           "lora_sgmv_fused_graph", "lora_status_string", "lora_last_error", "lora_version"]
NOALLOC_SCRATCH_BYTES = 16 << 20  # LORA_NOALLOC_SCRATCH_BYTES

_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m lora_adapter_batching_amd.build`")
    # torch (which provides the device memory and streams) brings its own HIP
    # runtime; loading it first makes the library bind to that same runtime,
    # so that one HIP runtime serves the process
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.lora_segments_from_ids.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, P]
    lib.lora_workspace_size.argtypes = [ctypes.c_int, ctypes.POINTER(CAdapters),
                                        ctypes.POINTER(CSegments), ctypes.POINTER(ctypes.c_size_t)]
    lib.lora_sgmv_shrink.argtypes = [P, I64, ctypes.POINTER(CAdapters), ctypes.POINTER(CSegments),
                                     P, I64, P, ctypes.c_size_t, P]
    lib.lora_sgmv_expand.argtypes = [P, I64, ctypes.POINTER(CAdapters), ctypes.POINTER(CSegments),
                                     P, I64, P, ctypes.c_size_t, P]
    lib.lora_sgmv_fused.argtypes = [P, I64, ctypes.POINTER(CAdapters), ctypes.POINTER(CSegments),
                                    P, I64, P, I64, P, ctypes.c_size_t, P]
    lib.lora_packed_backward.argtypes = [P, I64, P, I64, P, I64, ctypes.POINTER(CAdapters),
                                         ctypes.POINTER(CSegments), P, I64, P, P, ctypes.c_uint32,
                                         P, ctypes.c_size_t, P]
    lib.lora_workspace_size_multi.argtypes = [ctypes.c_int32, P, ctypes.POINTER(CSegments),
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.lora_sgmv_fused_multi.argtypes = [P, I64, ctypes.c_int32, P, ctypes.POINTER(CSegments), P, P,
                                          P, ctypes.c_size_t, P]
    lib.lora_sgmv_fused_noalloc.argtypes = [P, I64, ctypes.POINTER(CAdapters), ctypes.POINTER(CSegments),
                                            P, I64, P, I64, P]
    lib.lora_workspace_size_graph.argtypes = [ctypes.POINTER(CGraphAdapters), ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_size_t)]
    lib.lora_sgmv_fused_graph.argtypes = [P, I64, ctypes.POINTER(CGraphAdapters), P, ctypes.c_int32, P, I64,
                                          P, ctypes.c_size_t, P]
    lib.lora_status_string.restype = ctypes.c_char_p
    lib.lora_status_string.argtypes = [ctypes.c_int]
    lib.lora_last_error.restype = ctypes.c_char_p
    lib.lora_version.restype = ctypes.c_int
    for name in EXPORTS:
        if name not in ("lora_status_string", "lora_last_error", "lora_version"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != LORA_OK:
        lib = load()
        raise LoraError(status, lib.lora_last_error().decode())


def _ptr(t) -> int:
    """Device or host address of a torch tensor / numpy array (0 for None)."""
    if t is None:
        return 0
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Adapters:
    """Adapters resident on the GPU: device pointer tables + host ranks/scales.

    A, B: sequences of device bf16 tensors, A[i] [r_i, h_in], B[i] [h_out, r_i]
    (None allowed for rank 0). The pointer tables are int64 device tensors,
    so they can be rewritten in place between calls. With host_tables (the
    default) host copies of the tables go with every call too, and small
    launches take the addresses from them: after rewriting a device table in
    place, rewrite A_host / B_host (uint64 numpy arrays) the same way, or
    build the object with host_tables=False.
    """

    def __init__(self, A: Sequence, B: Sequence, ranks, scales, h_in: int, h_out: int,
                 device=None, host_tables: bool = True):
        import torch
        self.A, self.B = list(A), list(B)
        self.ranks = np.ascontiguousarray(ranks, dtype=np.int32)
        self.scales = np.ascontiguousarray(scales, dtype=np.float32)
        self.h_in, self.h_out = int(h_in), int(h_out)
        dev = device if device is not None else "cuda"
        self.A_ptrs = torch.tensor([_ptr(a) for a in self.A], dtype=torch.int64, device=dev)
        self.B_ptrs = torch.tensor([_ptr(b) for b in self.B], dtype=torch.int64, device=dev)
        self.A_host = np.array([_ptr(a) for a in self.A], dtype=np.uint64)
        self.B_host = np.array([_ptr(b) for b in self.B], dtype=np.uint64)
        self._c = CAdapters(len(self.ranks), self.h_in, self.h_out, _ptr(self.A_ptrs),
                            _ptr(self.B_ptrs), self.ranks.ctypes.data, self.scales.ctypes.data,
                            self.A_host.ctypes.data if host_tables else 0,
                            self.B_host.ctypes.data if host_tables else 0)

    @property
    def c(self):
        return ctypes.byref(self._c)


class Segments:
    """A batch in sorted-position order cut into one-adapter segments.

    seg_starts [S+1] and seg_adapter [S] are host arrays; token_rows is an
    optional int32 device tensor (row of x/y used by each sorted position);
    token_rows_host an optional int32 host array with the same rows (small
    forward launches carry it in their arguments; token_rows may then be
    None for them).
    """

    def __init__(self, seg_starts, seg_adapter, token_rows=None, token_rows_host=None):
        self.seg_starts = np.ascontiguousarray(seg_starts, dtype=np.int32)
        self.seg_adapter = np.ascontiguousarray(seg_adapter, dtype=np.int32)
        self.token_rows = token_rows
        S = int(self.seg_adapter.shape[0])
        T = int(self.seg_starts[-1]) if self.seg_starts.size else 0
        self.token_rows_host = None
        if token_rows_host is not None:
            self.token_rows_host = np.ascontiguousarray(token_rows_host, dtype=np.int32)
            if self.token_rows_host.shape != (T,):
                raise ValueError(f"token_rows_host must hold {T} rows, got shape {self.token_rows_host.shape}")
        self._c = CSegments(T, S, self.seg_starts.ctypes.data if S or self.seg_starts.size else 0,
                            self.seg_adapter.ctypes.data if S else 0, _ptr(token_rows),
                            self.token_rows_host.ctypes.data if self.token_rows_host is not None else 0)

    @property
    def num_tokens(self) -> int:
        return int(self._c.num_tokens)

    @property
    def c(self):
        return ctypes.byref(self._c)


def segments_from_ids(ids: np.ndarray, num_adapters: int):
    """Host bookkeeping: (perm [T], seg_starts [N+2], seg_adapter [N+1])."""
    lib = load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T = int(ids.shape[0])
    perm = np.zeros(max(T, 1), np.int32)
    starts = np.zeros(num_adapters + 2, np.int32)
    adap = np.zeros(num_adapters + 1, np.int32)
    _check(lib.lora_segments_from_ids(ids.ctypes.data if T else None, T, int(num_adapters),
                                      perm.ctypes.data, starts.ctypes.data, adap.ctypes.data))
    return perm[:T], starts, adap


def workspace_size(op: int, adapters: Adapters, segments: Optional[Segments] = None) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.lora_workspace_size(op, adapters.c, segments.c if segments is not None else None,
                                   ctypes.byref(n)))
    return int(n.value)


def new_workspace(op: int, adapters: Adapters, segments: Optional[Segments] = None, device="cuda"):
    """A zero-filled workspace tensor of the size `op` needs."""
    import torch
    n = workspace_size(op, adapters, segments)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def _ws(ws):
    if ws is None:
        return 0, 0
    return _ptr(ws), int(ws.numel() * ws.element_size())


def sgmv_shrink(x, adapters: Adapters, segments: Segments, u, ws=None, stream=None):
    lib = load()
    wp, wb = _ws(ws)
    _check(lib.lora_sgmv_shrink(_ptr(x), x.stride(0), adapters.c, segments.c, _ptr(u), u.stride(0),
                                wp, wb, _stream_handle(stream)))


def sgmv_expand(u, adapters: Adapters, segments: Segments, y, ws=None, stream=None):
    lib = load()
    wp, wb = _ws(ws)
    _check(lib.lora_sgmv_expand(_ptr(u), u.stride(0), adapters.c, segments.c, _ptr(y), y.stride(0),
                                wp, wb, _stream_handle(stream)))


def sgmv_fused(x, adapters: Adapters, segments: Segments, y, u_save=None, ws=None, stream=None):
    lib = load()
    wp, wb = _ws(ws)
    ldu = u_save.stride(0) if u_save is not None else 0
    _check(lib.lora_sgmv_fused(_ptr(x), x.stride(0), adapters.c, segments.c, _ptr(y), y.stride(0),
                               _ptr(u_save), ldu, wp, wb, _stream_handle(stream)))


def packed_backward(x, dy, u, adapters: Adapters, segments: Segments, dx, dA_ptrs, dB_ptrs,
                    flags: int = 0, ws=None, stream=None):
    """dA_ptrs / dB_ptrs: int64 device tensors of fp32 gradient addresses."""
    lib = load()
    wp, wb = _ws(ws)
    _check(lib.lora_packed_backward(
        _ptr(x), x.stride(0) if x is not None else 0, _ptr(dy), dy.stride(0) if dy is not None else 0,
        _ptr(u), u.stride(0) if u is not None else 0, adapters.c, segments.c, _ptr(dx),
        dx.stride(0) if dx is not None else 0, _ptr(dA_ptrs), _ptr(dB_ptrs), int(flags), wp, wb,
        _stream_handle(stream)))


def sgmv_fused_noalloc(x, adapters: Adapters, segments: Segments, y, u_save=None, stream=None):
    """lora_sgmv_fused_noalloc: the fused call with the library's static
    device scratch instead of a workspace."""
    lib = load()
    ldu = u_save.stride(0) if u_save is not None else 0
    _check(lib.lora_sgmv_fused_noalloc(_ptr(x), x.stride(0), adapters.c, segments.c, _ptr(y), y.stride(0),
                                       _ptr(u_save), ldu, _stream_handle(stream)))


class GraphAdapters:
    """Adapters described only by device tables (for lora_sgmv_fused_graph):
    int64 A/B pointer tables, int32 ranks and float32 scales, all device
    tensors the caller may rewrite between graph replays, plus the host bound
    max_rank."""

    def __init__(self, A_ptrs, B_ptrs, ranks, scales, h_in: int, h_out: int, max_rank: int):
        import torch
        n = int(ranks.numel())
        for name, t, dt in (("A_ptrs", A_ptrs, torch.int64), ("B_ptrs", B_ptrs, torch.int64),
                            ("ranks", ranks, torch.int32), ("scales", scales, torch.float32)):
            if not t.is_cuda or t.dtype != dt or not t.is_contiguous() or t.numel() != n:
                raise ValueError(f"{name} must be a contiguous {dt} device tensor of {n} entries")
        self.A_ptrs, self.B_ptrs, self.ranks, self.scales = A_ptrs, B_ptrs, ranks, scales
        self.h_in, self.h_out, self.max_rank = int(h_in), int(h_out), int(max_rank)
        self._c = CGraphAdapters(int(ranks.numel()), self.h_in, self.h_out, self.max_rank, _ptr(A_ptrs),
                                 _ptr(B_ptrs), _ptr(ranks), _ptr(scales))

    @property
    def c(self):
        return ctypes.byref(self._c)


def workspace_size_graph(adapters: GraphAdapters, num_tokens: int) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    _check(lib.lora_workspace_size_graph(adapters.c, int(num_tokens), ctypes.byref(n)))
    return int(n.value)


def new_workspace_graph(adapters: GraphAdapters, num_tokens: int, device="cuda"):
    import torch
    return torch.zeros(max(workspace_size_graph(adapters, num_tokens), 256), dtype=torch.uint8, device=device)


def sgmv_fused_graph(x, adapters: GraphAdapters, token_ids, y, ws, stream=None):
    """lora_sgmv_fused_graph: x, y in request order, token_ids an int32 device
    tensor of one adapter id per row of x."""
    import torch
    lib = load()
    T = int(token_ids.numel())
    if not token_ids.is_cuda or token_ids.dtype != torch.int32 or not token_ids.is_contiguous():
        raise ValueError("token_ids must be a contiguous int32 device tensor")
    for name, t, w in (("x", x, adapters.h_in), ("y", y, adapters.h_out)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or t.shape[0] < T or t.shape[1] != w or t.stride(1) != 1:
            raise ValueError(f"{name} must be a bf16 [>= {T}, {w}] matrix with unit column stride")
    wp, wb = _ws(ws)
    _check(lib.lora_sgmv_fused_graph(_ptr(x), x.stride(0), adapters.c, _ptr(token_ids), int(token_ids.numel()),
                                     _ptr(y), y.stride(0), wp, wb, _stream_handle(stream)))


def _multi_tables(adapters: Sequence[Adapters]):
    """C array of lora_adapters_t pointers (kept alive by the caller)."""
    arr = (ctypes.POINTER(CAdapters) * len(adapters))(*[ctypes.pointer(a._c) for a in adapters])
    return arr


def workspace_size_multi(adapters: Sequence[Adapters], segments: Segments) -> int:
    lib = load()
    n = ctypes.c_size_t(0)
    arr = _multi_tables(adapters)
    _check(lib.lora_workspace_size_multi(len(adapters), ctypes.cast(arr, ctypes.c_void_p), segments.c,
                                         ctypes.byref(n)))
    return int(n.value)


def new_workspace_multi(adapters: Sequence[Adapters], segments: Segments, device="cuda"):
    """A zero-filled workspace tensor for sgmv_fused_multi."""
    import torch
    return torch.zeros(max(workspace_size_multi(adapters, segments), 256), dtype=torch.uint8, device=device)


def sgmv_fused_multi(x, adapters: Sequence[Adapters], segments: Segments, ys: Sequence, ws=None, stream=None):
    """One launch for several projections over the same x: ys[p] +=
    s B_p,i (A_p,i x) with projection p's adapters."""
    import torch
    if len(ys) != len(adapters):
        raise ValueError(f"sgmv_fused_multi: {len(adapters)} adapter sets but {len(ys)} outputs")
    for p, y in enumerate(ys):
        if y.dtype != torch.bfloat16 or y.dim() != 2 or y.stride(1) != 1:
            raise ValueError(f"sgmv_fused_multi: ys[{p}] must be a 2-D bfloat16 tensor with unit column stride")
    lib = load()
    wp, wb = _ws(ws)
    arr = _multi_tables(adapters)
    yp = (ctypes.c_void_p * len(ys))(*[_ptr(y) for y in ys])
    ld = (ctypes.c_int64 * len(ys))(*[y.stride(0) for y in ys])
    _check(lib.lora_sgmv_fused_multi(_ptr(x), x.stride(0), len(adapters), ctypes.cast(arr, ctypes.c_void_p),
                                     segments.c, ctypes.cast(yp, ctypes.c_void_p),
                                     ctypes.cast(ld, ctypes.c_void_p), wp, wb, _stream_handle(stream)))


class CPlanItem(ctypes.Structure):
    """lora_plan_item_t of the internal inspection entry (csrc/lora_inspect.h)."""
    _fields_ = [(n, ctypes.c_int32) for n in
                ("launch", "phase", "block", "grid", "mode", "kind", "tile", "adapter", "proj", "rank",
                 "tok0", "ntok", "lo", "hi", "part", "aux")]


INSPECT_WITH_U, INSPECT_WITH_DX, INSPECT_ACCUMULATE = 1, 2, 4
PHASE_FWD, PHASE_WGRAD, PHASE_REDUCE, PHASE_TRANSPOSE, PHASE_PLAN = 0, 1, 2, 3, 4


def inspect_plan(op: int, adapters, segments: Segments, options: int = 0, cus: int = 256, xccs: int = 8):
    """Host-only listing of every workgroup the call `op` would launch
    (no GPU involved). adapters: one Adapters-like object, or a sequence of
    them for a multi-projection fused call. Returns (items, ranges): a numpy
    structured array with the lora_plan_item_t fields, and an int32 [n, 2]
    array of (first position, count) token ranges of weight-gradient jobs."""
    lib = load()
    fn = lib.lora_inspect_plan
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(CSegments), ctypes.c_uint32,
                   ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.POINTER(ctypes.c_int64), ctypes.c_void_p, ctypes.c_int64,
                   ctypes.POINTER(ctypes.c_int64)]
    ads = list(adapters) if isinstance(adapters, (list, tuple)) else [adapters]
    arr = _multi_tables(ads)
    n_items = ctypes.c_int64(0)
    n_ranges = ctypes.c_int64(0)
    cap, rcap = 1 << 14, 1 << 12
    while True:
        items = (CPlanItem * cap)()
        ranges = (ctypes.c_int32 * (2 * rcap))()
        _check(fn(op, len(ads), ctypes.cast(arr, ctypes.c_void_p), segments.c, options, cus, xccs,
                  ctypes.cast(items, ctypes.c_void_p), cap, ctypes.byref(n_items),
                  ctypes.cast(ranges, ctypes.c_void_p), rcap, ctypes.byref(n_ranges)))
        if n_items.value <= cap and n_ranges.value <= rcap:
            break
        cap = max(cap, int(n_items.value))
        rcap = max(rcap, int(n_ranges.value))
    dt = np.dtype([(f, np.int32) for f, _ in CPlanItem._fields_])
    out = np.frombuffer(bytes(items), dtype=dt, count=int(n_items.value)).copy()
    rg = np.frombuffer(bytes(ranges), dtype=np.int32, count=2 * int(n_ranges.value)).reshape(-1, 2).copy()
    return out, rg


def inspect_graph(num_adapters: int, h_in: int, h_out: int, max_rank: int, num_tokens: int, tiles: int,
                  cus: int = 256, xccs: int = 8):
    """Host-only listing of the workgroups of a device-planned call over
    num_tokens ids whose batch turns out to have `tiles` tiles (stand-in
    device tables, never dereferenced). Returns a numpy structured array with
    the lora_plan_item_t fields."""
    lib = load()
    fn = lib.lora_inspect_graph
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.POINTER(CGraphAdapters), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    fake = 1 << 40
    ga = CGraphAdapters(int(num_adapters), int(h_in), int(h_out), int(max_rank), fake, fake + 4096, fake + 8192,
                        fake + 12288)
    n = ctypes.c_int64(0)
    cap = 1 << 12
    while True:
        items = (CPlanItem * cap)()
        _check(fn(ctypes.byref(ga), int(num_tokens), int(tiles), int(cus), int(xccs), ctypes.cast(items, ctypes.c_void_p),
                  cap, ctypes.byref(n)))
        if n.value <= cap:
            break
        cap = int(n.value)
    dt = np.dtype([(f, np.int32) for f, _ in CPlanItem._fields_])
    return np.frombuffer(bytes(items), dtype=dt, count=int(n.value)).copy()


def version() -> int:
    return int(load().lora_version())
