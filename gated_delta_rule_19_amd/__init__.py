"""Gated DeltaNet-2 token-mixer core for AMD MI355X (gfx950).

Python face of the C ABI in ``include/gdn2.h`` (``libgdn2.so`` in this
directory): the chunked forward and the fused recurrent / decode step of the
GDN-2 recurrence (also over packed variable-length batches and with grouped
value heads), the output step, the short convolution of the prologue, with hand-written HIP kernels doing all the
arithmetic.
The library is loaded on first use; a missing library raises.
"""
from ._binding import (  # noqa: F401
    FLAG_GATE_LOGITS,
    FLAG_NEG_EIGVAL,
    FLAG_QK_L2NORM,
    CONV_SILU,
    Conv,
    Gdn2Error,
    Problem,
    abi_version,
    alloc_workspace,
    chunk_bwd,
    chunk_bwd_varlen,
    chunk_bwd_varlen_workspace_size,
    chunk_bwd_workspace_size,
    chunk_fwd,
    chunk_fwd_conv,
    chunk_fwd_noalloc,
    NOALLOC_SCRATCH_BYTES,
    chunk_fwd_varlen,
    chunk_fwd_varlen_workspace_size,
    chunk_fwd_workspace_size,
    chunk_prep,
    chunk_prep_workspace_size,
    chunk_state,
    gated_rmsnorm,
    lib,
    problem,
    recurrent_step,
    recurrent_step_conv,
    recurrent_step_gated,
    recurrent_varlen,
    short_conv,
    short_conv_bwd,
    short_conv_bwd_workspace_size,
    status_str,
)
