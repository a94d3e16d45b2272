"""Multi-adapter LoRA (SGMV shrink/expand, fused forward, packed backward)
for AMD MI355X (gfx950).

The compute path is the HIP library liblora_sgmv.so (C ABI in
include/lora_sgmv.h); this package holds its sources (csrc/), the build
script and a thin ctypes binding.
"""
from .binding import (  # noqa: F401
    Adapters,
    GraphAdapters,
    Segments,
    LoraError,
    GRAD_ACCUMULATE,
    OP_BACKWARD,
    OP_EXPAND,
    OP_FUSED,
    OP_SHRINK,
    load,
    new_workspace,
    new_workspace_graph,
    new_workspace_multi,
    packed_backward,
    segments_from_ids,
    sgmv_expand,
    sgmv_fused,
    sgmv_fused_graph,
    sgmv_fused_multi,
    sgmv_fused_noalloc,
    sgmv_shrink,
    version,
    workspace_size,
    workspace_size_graph,
    workspace_size_multi,
)
