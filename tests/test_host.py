"""Host-side checks that need no GPU: the C ABI exports, token bookkeeping
(bit-exact), host validation of every error path, and workspace sizing."""
import ctypes
import os
import re

import numpy as np
import pytest

import lora_adapter_batching_amd as L
from lora_adapter_batching_amd import binding as B
from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "lora_sgmv.h")).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*)\s+(lora_\w+)\s*\(", hdr, flags=re.M))
    assert {"lora_sgmv_shrink", "lora_sgmv_expand", "lora_sgmv_fused",
            "lora_packed_backward", "lora_segments_from_ids", "lora_workspace_size"} <= declared
    lib = L.load()
    for name in declared:
        assert hasattr(lib, name), name
    assert declared <= set(B.EXPORTS) | {"lora_version"}
    assert L.version() >= 100


def test_binding_structs_match_the_c_header(tmp_path):
    """Field offsets and sizes of the ctypes mirrors equal the C compiler's
    layout of lora_adapters_t and lora_segments_t."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    checks = []
    for cname, py in (("lora_adapters_t", B.CAdapters), ("lora_segments_t", B.CSegments),
                      ("lora_graph_adapters_t", B.CGraphAdapters)):
        checks.append((cname, "sizeof", f"sizeof({cname})", ctypes.sizeof(py)))
        for f, _ in py._fields_:
            checks.append((cname, f, f"offsetof({cname}, {f})", getattr(py, f).offset))
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"lora_sgmv.h\"\nint main(void) {\n"
    for _, _, expr, _ in checks:
        src += f'  printf("%zu\\n", (size_t)({expr}));\n'
    src += "  return 0;\n}\n"
    c = tmp_path / "layout.c"
    c.write_text(src)
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(c), "-o", str(exe)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    for (cname, f, _, want), g in zip(checks, got):
        assert g == want, f"{cname}.{f}: C {g}, ctypes {want}"


@pytest.mark.parametrize("seed", range(8))
def test_segments_from_ids_bit_exact(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 70))
    T = int(rng.integers(0, 5000))
    ids = rng.integers(-1, N, size=T).astype(np.int32)
    if seed % 3 == 0:
        ids[ids == N // 2] = 0  # force an empty segment
    perm, st, ad = L.segments_from_ids(ids, N)
    operm, ost, oad = oracle.segments_from_ids(ids, N)
    assert np.array_equal(perm, operm)
    assert np.array_equal(st, ost)
    assert np.array_equal(ad, oad)
    key = np.where(ids < 0, N, ids)
    assert np.array_equal(perm, np.argsort(key, kind="stable"))


def test_segments_from_ids_rejects_bad_ids():
    for bad in ([0, 5], [-2], [3, 0, 4]):
        with pytest.raises(B.LoraError) as e:
            L.segments_from_ids(np.array(bad, np.int32), 4)
        assert e.value.status == B.LORA_INVALID_ARGUMENT
    with pytest.raises(B.LoraError):
        L.segments_from_ids(np.array([0], np.int32), 0)


# ---------------------------------------------------------------------------
# Validation (host mirrors only; the calls below never reach the GPU)
# ---------------------------------------------------------------------------
FAKE = 1 << 20  # a 16-byte aligned non-null "device" address, never dereferenced


def _adapters(ranks=(8, 16), scales=None, h_in=64, h_out=32, A=FAKE, Bp=FAKE):
    ranks = np.ascontiguousarray(ranks, np.int32)
    scales = np.ascontiguousarray(scales if scales is not None else [1.0] * len(ranks), np.float32)
    c = B.CAdapters(len(ranks), h_in, h_out, A, Bp, ranks.ctypes.data, scales.ctypes.data)
    return c, (ranks, scales)


def _segments(starts, adapter, T=None, token_rows=0, token_rows_host=0):
    starts = np.ascontiguousarray(starts, np.int32)
    adapter = np.ascontiguousarray(adapter, np.int32)
    T = int(starts[-1]) if T is None else T
    c = B.CSegments(T, len(adapter), starts.ctypes.data, adapter.ctypes.data if len(adapter) else 0,
                    token_rows, token_rows_host)
    return c, (starts, adapter)


def _fused(ad, sg, x=FAKE, ldx=64, y=FAKE, ldy=32, u=0, ldu=0, ws=FAKE, wsb=1 << 30):
    lib = L.load()
    return lib.lora_sgmv_fused(x, ldx, ctypes.byref(ad), ctypes.byref(sg), y, ldy, u, ldu, ws, wsb, 0)


def test_validation_error_codes():
    lib = L.load()
    ad, keep_a = _adapters()
    sg, keep_s = _segments([0, 3, 5], [0, 1])
    cases = []
    # segment metadata (the tuples keep the host arrays alive)
    cases.append((_segments([1, 3, 5], [0, 1]), "seg_starts[0]"))
    cases.append((_segments([0, 4, 3], [0, 1], T=3), "decreases"))
    cases.append((_segments([0, 3, 5], [0, 2]), "outside"))
    cases.append((_segments([0, 3, 5], [-2, 0]), "outside"))
    cases.append((_segments([0, 3, 5], [0, 1], T=6), "differs"))
    for (seg, _keep), msg in cases:
        st = _fused(ad, seg)
        assert st == B.LORA_INVALID_ARGUMENT, msg
        assert msg in lib.lora_last_error().decode()
    # adapters
    a_bad, k1 = _adapters(ranks=(8, 129))
    assert _fused(a_bad, sg) == B.LORA_UNSUPPORTED
    a_bad, k2 = _adapters(ranks=(8, -1))
    assert _fused(a_bad, sg) == B.LORA_INVALID_ARGUMENT
    a_bad, k3 = _adapters(scales=[1.0, float("nan")])
    assert _fused(a_bad, sg) == B.LORA_INVALID_ARGUMENT
    a_bad, k4 = _adapters(h_in=60)
    assert _fused(a_bad, sg) == B.LORA_INVALID_ARGUMENT
    a_bad, k5 = _adapters(A=0)
    assert _fused(a_bad, sg) == B.LORA_INVALID_ARGUMENT
    # rows, strides, alignment
    assert _fused(ad, sg, x=0) == B.LORA_INVALID_ARGUMENT
    assert _fused(ad, sg, x=FAKE + 2) == B.LORA_INVALID_ARGUMENT
    assert _fused(ad, sg, ldx=60) == B.LORA_INVALID_ARGUMENT
    assert _fused(ad, sg, ldx=68) == B.LORA_INVALID_ARGUMENT
    assert _fused(ad, sg, ldy=16) == B.LORA_INVALID_ARGUMENT
    assert _fused(ad, sg, u=FAKE, ldu=8) == B.LORA_INVALID_ARGUMENT  # below rank 16
    assert _fused(ad, sg, u=FAKE + 2, ldu=16) == B.LORA_INVALID_ARGUMENT
    # workspace
    need = ctypes.c_size_t(0)
    assert lib.lora_workspace_size(B.OP_FUSED, ctypes.byref(ad), ctypes.byref(sg), ctypes.byref(need)) == 0
    assert need.value > 0
    assert _fused(ad, sg, wsb=need.value - 1) == B.LORA_WORKSPACE_TOO_SMALL
    assert _fused(ad, sg, ws=0) == B.LORA_INVALID_ARGUMENT
    assert _fused(ad, sg, ws=FAKE + 16) == B.LORA_INVALID_ARGUMENT
    # nothing to do: every segment skipped -> OK without touching the GPU
    sg_skip, k6 = _segments([0, 3, 5], [-1, -1])
    assert _fused(ad, sg_skip, x=0, y=0) == B.LORA_OK
    a_r0, k7 = _adapters(ranks=(0, 0))
    assert _fused(a_r0, sg, x=0, y=0) == B.LORA_OK


def test_backward_validation():
    lib = L.load()
    ad, ka = _adapters()
    sg, ks = _segments([0, 3, 5], [0, 1])
    n = ctypes.c_size_t(0)
    assert lib.lora_workspace_size(B.OP_BACKWARD, ctypes.byref(ad), ctypes.byref(sg), ctypes.byref(n)) == 0

    def bwd(flags=0, dA=FAKE, dB=FAKE, x=FAKE, dy=FAKE, dx=FAKE, wsb=n.value):
        return lib.lora_packed_backward(x, 64, dy, 32, 0, 0, ctypes.byref(ad), ctypes.byref(sg), dx, 64,
                                        dA, dB, flags, FAKE, wsb, 0)

    assert bwd(flags=2) == B.LORA_INVALID_ARGUMENT
    assert bwd(dA=0) == B.LORA_INVALID_ARGUMENT
    assert bwd(dy=0) == B.LORA_INVALID_ARGUMENT
    assert bwd(dx=FAKE + 8) == B.LORA_INVALID_ARGUMENT
    assert bwd(wsb=n.value - 1) == B.LORA_WORKSPACE_TOO_SMALL


def test_workspace_size_bounds():
    lib = L.load()
    sizes = {}
    for T in (16, 4096, 65536):
        ad, ka = _adapters(ranks=(8, 64, 32), h_in=3584, h_out=3584)
        sg, ks = _segments([0, T], [1])
        for op in (B.OP_SHRINK, B.OP_EXPAND, B.OP_FUSED, B.OP_BACKWARD):
            n = ctypes.c_size_t(0)
            assert lib.lora_workspace_size(op, ctypes.byref(ad), ctypes.byref(sg), ctypes.byref(n)) == 0
            sizes[(T, op)] = n.value
    assert sizes[(16, B.OP_EXPAND)] == 0
    # forward workspaces grow with the batch's tile count up to a fixed cap
    # (2048 split-shrink parts of 32 x 64 fp32 here, plus 260 KiB of hand-off
    # words: 4 KiB of counters, then 2048 stamps on 128-byte lines)
    cap = 2048 * 32 * 64 * 4 + 260 * 1024
    assert sizes[(16, B.OP_FUSED)] < sizes[(4096, B.OP_FUSED)] == sizes[(65536, B.OP_FUSED)] <= cap + 512
    assert sizes[(16, B.OP_BACKWARD)] < sizes[(65536, B.OP_BACKWARD)]
    n = ctypes.c_size_t(0)
    assert lib.lora_workspace_size(7, ctypes.byref(ad), ctypes.byref(sg), ctypes.byref(n)) != 0


def test_multi_projection_validation():
    """lora_sgmv_fused_multi / lora_workspace_size_multi reject malformed
    requests on the host mirrors before any GPU call."""
    lib = L.load()
    a0, k0 = _adapters(ranks=(8, 16), h_in=64, h_out=32)
    a1, k1 = _adapters(ranks=(4, 0), h_in=64, h_out=48)
    a_hin, k2 = _adapters(ranks=(8, 16), h_in=72, h_out=32)
    a_n, k3 = _adapters(ranks=(8, 16, 8), h_in=64, h_out=32)
    sg, ks = _segments([0, 3, 5], [0, 1])

    def arr(*ads):
        return (ctypes.POINTER(B.CAdapters) * len(ads))(*[ctypes.pointer(a) for a in ads])

    def call(ads, n=None, ys=None, lds=None, ws=FAKE, wsb=1 << 30):
        n = len(ads) if n is None else n
        ys = ys if ys is not None else [FAKE + (1 << 24) * (p + 1) for p in range(len(ads))]
        lds = lds if lds is not None else [32, 48, 32, 32][:len(ads)]
        yp = (ctypes.c_void_p * len(ys))(*ys)
        ld = (ctypes.c_int64 * len(lds))(*lds)
        return lib.lora_sgmv_fused_multi(FAKE, 64, n, ctypes.cast(arr(*ads), ctypes.c_void_p), ctypes.byref(sg),
                                         ctypes.cast(yp, ctypes.c_void_p), ctypes.cast(ld, ctypes.c_void_p),
                                         ws, wsb, 0)

    assert call([a0, a1], n=0) == B.LORA_INVALID_ARGUMENT
    assert call([a0, a1], n=5) == B.LORA_INVALID_ARGUMENT
    assert call([a0, a_hin]) == B.LORA_INVALID_ARGUMENT
    assert "same num_adapters and h_in" in lib.lora_last_error().decode()
    assert call([a0, a_n]) == B.LORA_INVALID_ARGUMENT
    assert call([a0, a1], ys=[FAKE, 0]) == B.LORA_INVALID_ARGUMENT  # projection 1 has work (adapter 0)
    assert call([a0, a1], lds=[32, 40]) == B.LORA_INVALID_ARGUMENT  # row stride below h_out 48
    # outputs that alias each other or x are refused
    assert call([a0, a1], ys=[FAKE + 4096, FAKE + 4096]) == B.LORA_INVALID_ARGUMENT
    assert "same buffer" in lib.lora_last_error().decode()
    assert call([a0, a1], ys=[FAKE + 4096, FAKE]) == B.LORA_INVALID_ARGUMENT
    assert "overlap x" in lib.lora_last_error().decode()
    n = ctypes.c_size_t(0)
    assert lib.lora_workspace_size_multi(2, ctypes.cast(arr(a0, a1), ctypes.c_void_p), ctypes.byref(sg),
                                         ctypes.byref(n)) == 0
    n1 = ctypes.c_size_t(0)
    assert lib.lora_workspace_size_multi(1, ctypes.cast(arr(a0), ctypes.c_void_p), ctypes.byref(sg),
                                         ctypes.byref(n1)) == 0
    assert n.value >= n1.value > 0
    assert call([a0, a1], wsb=n.value - 1) == B.LORA_WORKSPACE_TOO_SMALL
    # nothing to do: every segment skipped -> OK without touching the GPU
    sg_skip, k4 = _segments([0, 3, 5], [-1, -1])
    yp = (ctypes.c_void_p * 2)(0, 0)
    ld = (ctypes.c_int64 * 2)(32, 48)
    assert lib.lora_sgmv_fused_multi(0, 64, 2, ctypes.cast(arr(a0, a1), ctypes.c_void_p), ctypes.byref(sg_skip),
                                     ctypes.cast(yp, ctypes.c_void_p), ctypes.cast(ld, ctypes.c_void_p),
                                     0, 0, 0) == B.LORA_OK


def test_token_rows_gather_span_is_checked_on_the_host():
    """With a token-row table the kernels reach every row through one window
    of 2 GiB - 16 bytes from the matrix base; a batch whose T distinct rows
    cannot fit in it is refused before any GPU call, for every matrix the
    call touches (x, y, dx, dy)."""
    lib = L.load()
    span = 0x7FFFFFF0
    h = 19456  # gate_up-like output width: rows of 38912 bytes
    T_fit = (span // 2 - h) // h + 1       # largest T whose rows fit
    for T, ok in ((T_fit, True), (T_fit + 1, False)):
        ad, ka = _adapters(ranks=(16, 8), h_in=64, h_out=h)
        sg, ks = _segments([0, T], [0], token_rows=FAKE)
        # a zero-byte workspace stops a call that passes every argument check
        # at the workspace check, which runs after the gather check and
        # before anything reaches the GPU
        st = _fused(ad, sg, ldx=64, ldy=h, wsb=0)
        if ok:
            assert st == B.LORA_WORKSPACE_TOO_SMALL, lib.lora_last_error().decode()
        else:
            assert st == B.LORA_INVALID_ARGUMENT
            assert "gather limit" in lib.lora_last_error().decode()
    # the same rows without a table address x/y per tile: no such limit
    ad, ka = _adapters(ranks=(16, 8), h_in=64, h_out=h)
    sg, ks = _segments([0, T_fit + 1], [0])
    assert _fused(ad, sg, ldx=64, ldy=h, wsb=0) == B.LORA_WORKSPACE_TOO_SMALL
    # an input-side stride alone can trip it too (x in a shrink, dy in a backward)
    T = 1 << 16
    ad, ka = _adapters(ranks=(16, 8), h_in=16384, h_out=32)
    sg, ks = _segments([0, T], [0], token_rows=FAKE)
    u = FAKE
    st = lib.lora_sgmv_shrink(FAKE, 16384, ctypes.byref(ad), ctypes.byref(sg), u, 16, FAKE, 0, 0)
    assert st == B.LORA_INVALID_ARGUMENT and "x: with token_rows" in lib.lora_last_error().decode()
    ad, ka = _adapters(ranks=(16, 8), h_in=64, h_out=16384)
    st = lib.lora_packed_backward(FAKE, 64, FAKE, 16384, 0, 0, ctypes.byref(ad), ctypes.byref(sg), 0, 0,
                                  FAKE, FAKE, 0, FAKE, 0, 0)
    assert st == B.LORA_INVALID_ARGUMENT and "dy: with token_rows" in lib.lora_last_error().decode()


def test_host_row_copy_alone_serves_only_small_launches():
    """A call given only the host copy of the row table (no device table) must
    fit in one small launch (at most 16 segments, 256 tokens), which carries
    the rows; larger ones, and every backward, are refused before any GPU
    call. With both tables given, large calls use the device one."""
    lib = L.load()
    rows = np.arange(400, dtype=np.int32)
    host = rows.ctypes.data

    def fused(T, n_seg, token_rows=0, token_rows_host=host):
        cuts = np.linspace(0, T, n_seg + 1).astype(np.int32)
        ad, ka = _adapters(ranks=[8] * n_seg, h_in=64, h_out=32)
        sg, ks = _segments(cuts, np.arange(n_seg, dtype=np.int32), token_rows=token_rows,
                           token_rows_host=token_rows_host)
        # a zero-byte workspace stops a call that passes every argument check
        return _fused(ad, sg, wsb=0), (ad, ka, sg, ks)

    assert fused(256, 16)[0] == B.LORA_WORKSPACE_TOO_SMALL, lib.lora_last_error().decode()
    for T, n_seg in ((257, 2), (64, 17)):
        st, keep = fused(T, n_seg)
        assert st == B.LORA_INVALID_ARGUMENT
        assert "host copy alone" in lib.lora_last_error().decode()
        st, keep = fused(T, n_seg, token_rows=FAKE)
        assert st == B.LORA_WORKSPACE_TOO_SMALL, lib.lora_last_error().decode()
    # shrink-only: the same limit
    ad, ka = _adapters(ranks=(16, 8), h_in=64, h_out=32)
    sg, ks = _segments([0, 150, 300], [0, 1], token_rows_host=host)
    st = lib.lora_sgmv_shrink(FAKE, 64, ctypes.byref(ad), ctypes.byref(sg), FAKE, 16, FAKE, 0, 0)
    assert st == B.LORA_INVALID_ARGUMENT and "host copy alone" in lib.lora_last_error().decode()
    # the backward reads rows in kernels that take no plan rows
    sg, ks = _segments([0, 3, 5], [0, 1], token_rows_host=host)
    st = lib.lora_packed_backward(FAKE, 64, FAKE, 32, 0, 0, ctypes.byref(ad), ctypes.byref(sg), 0, 0,
                                  FAKE, FAKE, 0, FAKE, 1 << 30, 0)
    assert st == B.LORA_INVALID_ARGUMENT and "device memory" in lib.lora_last_error().decode()


def test_noalloc_refuses_batches_beyond_its_static_scratch():
    """lora_sgmv_fused_noalloc checks the batch's workspace need against its
    static scratch before any HIP call (so this runs without a GPU)."""
    lib = L.load()
    assert B.NOALLOC_SCRATCH_BYTES == 16 << 20
    T = 65536
    ad, ka = _adapters(ranks=(128, 8), h_in=4096, h_out=4096)
    sg, ks = _segments([0, T], [0])
    need = ctypes.c_size_t(0)
    assert lib.lora_workspace_size(B.OP_FUSED, ctypes.byref(ad), ctypes.byref(sg), ctypes.byref(need)) == 0
    assert need.value > B.NOALLOC_SCRATCH_BYTES
    st = lib.lora_sgmv_fused_noalloc(FAKE, 4096, ctypes.byref(ad), ctypes.byref(sg), FAKE + (1 << 30), 4096,
                                     0, 0, 0)
    assert st == B.LORA_UNSUPPORTED
    assert "static scratch" in lib.lora_last_error().decode()
    # argument errors come first, as for lora_sgmv_fused
    assert lib.lora_sgmv_fused_noalloc(0, 4096, ctypes.byref(ad), ctypes.byref(sg), FAKE, 4096, 0, 0, 0) \
        == B.LORA_INVALID_ARGUMENT


def test_graph_call_validation():
    """lora_sgmv_fused_graph / lora_workspace_size_graph check their host
    arguments before any HIP call (a zero-byte workspace stops a valid call
    at the workspace check, so nothing reaches the GPU here)."""
    lib = L.load()

    def ga(N=8, h_in=64, h_out=32, max_rank=32, tabs=FAKE):
        return B.CGraphAdapters(N, h_in, h_out, max_rank, tabs, tabs, tabs, tabs)

    def call(a, T=16, x=FAKE, ldx=64, y=FAKE + (1 << 24), ldy=32, ids=FAKE, wsb=0):
        return lib.lora_sgmv_fused_graph(x, ldx, ctypes.byref(a), ids, T, y, ldy, FAKE, wsb, 0)

    n = ctypes.c_size_t(0)
    assert lib.lora_workspace_size_graph(ctypes.byref(ga()), 256, ctypes.byref(n)) == 0 and n.value > 0
    n2 = ctypes.c_size_t(0)
    assert lib.lora_workspace_size_graph(ctypes.byref(ga()), 16, ctypes.byref(n2)) == 0 and n2.value < n.value
    assert call(ga()) == B.LORA_WORKSPACE_TOO_SMALL  # every argument valid
    assert call(ga(), T=0) == B.LORA_OK                # nothing to do
    assert call(ga(N=0)) == B.LORA_INVALID_ARGUMENT
    assert call(ga(N=257)) == B.LORA_INVALID_ARGUMENT
    assert call(ga(max_rank=129)) == B.LORA_UNSUPPORTED
    assert call(ga(max_rank=0)) == B.LORA_INVALID_ARGUMENT
    assert call(ga(h_in=60)) == B.LORA_INVALID_ARGUMENT
    assert call(ga(tabs=0)) == B.LORA_INVALID_ARGUMENT
    assert call(ga(), T=-1) == B.LORA_INVALID_ARGUMENT
    assert call(ga(), ids=0) == B.LORA_INVALID_ARGUMENT
    assert call(ga(), x=FAKE + 2) == B.LORA_INVALID_ARGUMENT
    assert call(ga(), ldy=16) == B.LORA_INVALID_ARGUMENT
    assert call(ga(), y=FAKE) == B.LORA_INVALID_ARGUMENT  # y is x
    # rows 0 .. T-1 must fit the 2 GiB gather window
    assert call(ga(h_out=19456), T=60000, ldy=19456) == B.LORA_INVALID_ARGUMENT
    assert "gather limit" in lib.lora_last_error().decode()
