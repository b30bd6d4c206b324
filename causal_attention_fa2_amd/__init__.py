"""MI355X (gfx950) causal / sliding-window grouped-query attention, forward and backward.

The computation runs in hand-written HIP kernels behind the C ABI of libattn.so
(include/attn.h); this package is its thin ctypes binding. Importing it loads nothing; the
library is loaded on first use and every call raises if it is missing.
"""
from ._binding import (  # noqa: F401
    ATTN_BF16, ATTN_ERR_DEVICE, ATTN_ERR_INVALID, ATTN_ERR_SCRATCH, ATTN_ERR_UNSUPPORTED, ATTN_F32,
    ATTN_NOALLOC_SCRATCH_BYTES, ATTN_OK, LIB_PATH,
    AttnError, attn_abi_version, attn_bwd, attn_bwd_qk, attn_bwd_qk_noalloc, attn_bwd_qk_workspace_bytes,
    attn_bwd_qk_workspace_bytes_for, attn_decode_fwd,
    attn_decode_workspace_bytes,
    attn_bwd_varlen, attn_bwd_workspace_bytes, attn_fwd, attn_fwd_paged, attn_fwd_qk, attn_fwd_varlen,
    attn_set_launch_hook, attn_status_string, backward,
    forward, load_library, status_string,
)
