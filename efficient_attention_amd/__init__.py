"""Kernelized linear attention (phi = elu + 1, or FAVOR+ random features) for AMD Instinct
MI355X (gfx950).

The computation lives in hand-written HIP kernels behind the C ABI of include/linattn.h
(liblinattn.so, built in-tree by ``python -m efficient_attention_amd.build``).  This package
only marshals torch tensors and streams into that library; it has no other code path.
"""
from ._binding import (  # noqa: F401
    EXPORTS,
    LA_DTYPE_BF16,
    LA_DTYPE_F32,
    LIB_PATH,
    LinAttnError,
    la_abi_version,
    la_causal_plan,
    la_causal_segments,
    la_causal_workspace_bytes,
    la_ceiling_causal_pattern,
    la_ceiling_copy,
    la_ceiling_read,
    la_decode_step,
    la_decode_step_masked,
    la_favor_causal_workspace_bytes,
    la_favor_decode_step,
    la_favor_forward_causal,
    la_favor_forward_noncausal,
    la_favor_noncausal_workspace_bytes,
    la_forward_causal,
    la_forward_causal_state,
    la_forward_causal_varlen,
    la_forward_noncausal,
    la_forward_noncausal_noalloc,
    LA_NOALLOC_SCRATCH_BYTES,
    la_forward_noncausal_varlen,
    la_noncausal_varlen_workspace_bytes,
    la_causal_varlen_workspace_bytes,
    la_noncausal_workspace_bytes,
    la_state_sums,
    la_state_sums_workspace_bytes,
    la_status_string,
    load,
    release_workspaces,
)
