"""Blockwise ring attention, per-device hot path, for MI355X (gfx950).

A thin Python binding over the C ABI of ``libringattn.so`` (declared in ``include/ring_attn.h``):
the functions here only marshal arguments (torch tensors to device pointers, streams to handles)
and turn status codes into exceptions.  Every step of the computation runs in the HIP kernels.
There is no CPU fallback: the functions raise if the library is not built or no GPU is present.
"""
from ._binding import (  # noqa: F401
    RA_BF16, RA_F32, RA_LAYOUT_CONTIGUOUS, RA_LAYOUT_STRIPED, RA_LAYOUT_ZIGZAG, RA_MASK_CAUSAL, RA_MASK_NONE,
    RA_MAX_D, RA_MAX_DEV, RA_STEP_INIT, RA_BWD_INIT_DQ, RA_BWD_INIT_DKV, RingAttnError, HipEvent, lib, lib_path, ring_attn_finalize, ring_attn_local,
    ring_attn_local_workspace_bytes, ring_attn_plan, ring_attn_step, ring_attn_strerror, ring_attn_visible_pairs,
    ring_attn_bwd_prep, ring_attn_bwd_step, ring_attn_bwd_local, ring_attn_bwd_local_workspace_bytes,
    RA_FFN_GELU, RA_FFN_RELU, ring_attn_ffn, ring_attn_ffn_workspace_bytes,
    EXPORTED_SYMBOLS, RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP, RA_ERR_WORKSPACE, RA_ERR_INJECTED,
    RA_ERR_SCRATCH, ring_attn_local_noalloc, ring_attn_noalloc_scratch_bytes,
)
