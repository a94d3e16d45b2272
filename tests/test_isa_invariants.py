"""Invariants of the compiled gfx950 code that the kernels rely on (CPU only:
hipcc cross-compiles the device code to assembly; no GPU needed).

- The shrink's LDS-destination loads are inline assembly that sets M0 to the
  LDS address: every such M0 source and buffer descriptor must be a scalar
  register, and the compiler must not use M0 anywhere else.
- No kernel spills to scratch memory (a spill would also add vector memory
  operations that the explicit load counts of the shrink do not expect).
- The output rows y are streamed: every 16-byte buffer store of the forward
  kernels (the y stores) carries the non-temporal bit, and so do the x loads
  of one-item-per-tile launches (a second form of the LDS-destination load).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lora_adapter_batching_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def _device_asm(src, tmp_path):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / (os.path.basename(src) + ".s")
    from lora_adapter_batching_amd.build import CODEGEN_FLAGS
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc"] + CODEGEN_FLAGS + [
        "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S", "-o", str(out), src]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


@pytest.fixture(scope="module")
def fwd_asm(tmp_path_factory):
    return _device_asm(os.path.join(CSRC, "lora_fwd.hip"), tmp_path_factory.mktemp("asm"))


@pytest.fixture(scope="module")
def bwd_asm(tmp_path_factory):
    return _device_asm(os.path.join(CSRC, "lora_bwd.hip"), tmp_path_factory.mktemp("asm"))


def test_lds_loads_use_scalar_m0_and_descriptor(fwd_asm):
    lines = fwd_asm.splitlines()
    n_loads = n_stream = 0
    in_asm = False
    for i, l in enumerate(lines):
        s = l.split(";")[0].strip()
        if "ASMSTART" in l:
            in_asm = True
            continue
        if "ASMEND" in l:
            in_asm = False
            continue
        if not s:
            continue
        if in_asm:
            m = re.match(r"s_mov_b32 m0, (\S+)", s)
            if m:
                assert re.fullmatch(r"s\d+", m.group(1)), f"line {i}: M0 from {m.group(1)}"
            m = re.match(r"buffer_load_dwordx4 v\d+, (\S+), 0 offen( nt)? lds", s)
            if m:
                n_loads += 1
                n_stream += m.group(2) is not None
                assert re.fullmatch(r"s\[\d+:\d+\]", m.group(1)), f"line {i}: descriptor {m.group(1)}"
        else:
            assert not re.search(r"\bm0\b", s), f"line {i}: compiler use of M0: {s}"
    assert n_loads > 0
    assert 0 < n_stream < n_loads, (n_stream, n_loads)


def test_output_row_stores_are_streamed(fwd_asm):
    stores = [l.split(";")[0].strip() for l in fwd_asm.splitlines() if "buffer_store_dwordx4" in l]
    assert stores
    plain = [s for s in stores if not re.search(r"\bnt\b", s)]
    assert not plain, plain[:3]


def test_no_scratch(fwd_asm, bwd_asm):
    for text in (fwd_asm, bwd_asm):
        sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", text)
        assert sizes and all(int(v) == 0 for v in sizes), sizes


def test_part_loads_are_whole_device_scope_vectors(fwd_asm):
    """The split hand-off sums its parts from 16-byte device-scope loads:
    every forward kernel instance has some, and no part is read with
    narrower device-scope loads (a bit cast of a vector element once turned
    the vector loads into single-word reads of element 0)."""
    kernels = re.split(r"\n(?=_ZN4lora15sgmv_fwd_kernel\S*:)", fwd_asm)
    n = 0
    for k in kernels:
        if not k.startswith("_ZN4lora15sgmv_fwd_kernel"):
            continue
        body = k.split(".Lfunc_end")[0]
        n += 1
        assert re.search(r"buffer_load_dwordx4 .*\bsc1\b", body), k.split(":")[0]
        assert not re.search(r"buffer_load_dword v\d+, .*\bsc1\b", body), k.split(":")[0]
    assert n > 0
