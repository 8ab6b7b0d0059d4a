"""MI355X (gfx950) chunkwise gated delta rule: forward, decode step, backward.

The computation lives in hand-written HIP kernels behind the C ABI of
include/gdn.h (libgdn.so, built by `python -m gated_delta_rule_14_amd.build`);
this package is a thin binding over it.  Loading is lazy: importing works
without a GPU, every compute call needs the built library and a device.
"""
from ._binding import (ABI_VERSION, EXPORTS, LIB_PATH, Activation, FwdDesc, GdnError,  # noqa: F401
                       StepDesc, WorkspaceLayout, activation, bwd_workspace_bytes, chunk_bwd,
                       chunk_fwd, chunk_intra, chunk_scan, fwd_desc, load, recurrent_step,
                       seqlens_status, sync_status, sync_status_offset, workspace_bytes,
                       workspace_layout)

__all__ = ["load", "activation", "chunk_fwd", "chunk_bwd", "chunk_intra", "chunk_scan",
           "recurrent_step", "workspace_bytes", "bwd_workspace_bytes", "workspace_layout",
           "fwd_desc", "seqlens_status", "sync_status", "sync_status_offset", "GdnError",
           "LIB_PATH", "EXPORTS"]
