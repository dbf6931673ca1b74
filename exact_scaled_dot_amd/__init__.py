"""libsdpa: exact scaled dot-product attention (forward, decode, paged, backward) on MI355X (gfx950).

The computation lives in the HIP library libsdpa.so (include/sdpa.h); this
package is its thin ctypes binding plus the seeded workload generator.
"""

from .sdpa import (  # noqa: F401
    MASK_CAUSAL, MASK_KEY_PADDING, MASK_NONE, MAX_SPLITS, NOALLOC_SCRATCH_BYTES, SDPA_BF16, SDPA_ERR_HIP,
    SDPA_ERR_INVALID_ARGUMENT, SDPA_ERR_UNSUPPORTED, SDPA_ERR_WORKSPACE, SDPA_F16, SDPA_F32, SDPA_OK,
    SdpaError, decode_workspace_views, last_error, load_library, sdpa_backward, sdpa_backward_bias,
    sdpa_backward_atomic_workspace_size, sdpa_backward_workspace_size, sdpa_block_forward,
    sdpa_block_workspace_size, sdpa_decode, sdpa_decode_noalloc, sdpa_decode_workspace_size, sdpa_forward,
    sdpa_forward_bias, sdpa_forward_lse, sdpa_paged_attention, sdpa_paged_backward,
    sdpa_paged_backward_workspace_size, sdpa_paged_prefill, status_string,
)
