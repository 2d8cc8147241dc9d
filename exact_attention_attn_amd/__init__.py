"""Exact attention forward for AMD Instinct MI355X (gfx950).

The computation lives in ``libattn.so`` (hand-written HIP kernels behind the C ABI of
``include/attn.h``).  This package is its thin Python binding: the functions below
have the same names as the C entry points and only marshal arguments.  PyTorch is
used for device memory and streams.
"""
from ._lib import (  # noqa: F401
    ATTN_DTYPE_BF16,
    ATTN_DTYPE_F32,
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_LAUNCH,
    ATTN_ERR_SCRATCH_LIMIT,
    ATTN_ERR_UNSUPPORTED,
    ATTN_OK,
    EXPORTS,
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    AttnError,
    attn_bwd,
    attn_bwd_workspace_size,
    attn_bwd_varlen,
    attn_bwd_varlen_workspace_size,
    attn_decode_paged,
    attn_decode_paged_noalloc,
    attn_decode_paged_workspace_size,
    attn_fwd,
    attn_fwd_varlen,
    attn_store_kvcache,
    load,
    status_string,
)
