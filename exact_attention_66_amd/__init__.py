"""Exact tiled attention with online softmax for AMD MI355X (gfx950).

The computation lives in libattn.so (hand-written HIP kernels behind the C
ABI of include/attn.h); this package only loads it and marshals torch tensors
into its calls.  Build the library with ``python -m exact_attention_66_amd.build``.
"""
from ._binding import (  # noqa: F401
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_FP16,
    ATTN_OK,
    EXPORTED,
    KERNEL_KINDS,
    LIB_PATH,
    STATUS_NAMES,
    AttnError,
    attn_bwd,
    attn_bwd_strided_workspace_bytes,
    attn_bwd_workspace_bytes,
    attn_fwd,
    attn_fwd_kvcache,
    attn_fwd_kvcache_noalloc,
    ATTN_KV_SCRATCH_BYTES,
    attn_fwd_kvcache_splits,
    attn_fwd_kvcache_workspace_bytes,
    attn_last_hip_error,
    attn_profile_start,
    attn_profile_stop,
    attn_status_string,
    backward,
    default_scale,
    forward,
    forward_kvcache,
    forward_alibi,
    backward_alibi,
    forward_kvcache_alibi,
    forward_kvcache_gqa,
    attn_fwd_kvcache_gqa_workspace_bytes,
    dropout_threshold,
    forward_dropout,
    backward_dropout,
    dropout_draws,
    load,
)
