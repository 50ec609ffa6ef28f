"""Attention over a paged KV cache on MI355X (gfx950): Python face of libpa.

All computation runs in libpa.so (hand-written HIP kernels and a C++ host
allocator behind a C ABI, see include/pa.h).  This package only marshals
arguments; importing it fails when the library has not been built.
"""
from ._binding import (  # noqa: F401
    BLOCK, EXPORTS, LIB_PATH, PA_ALLOC_LATER, PA_ALLOC_NEVER, PA_ALLOC_OK, PA_BF16, PA_DEV_BAD_BLOCK,
    PA_DEV_BAD_GROUP, PA_DEV_BAD_LENGTH, PA_DEV_BAD_POSITION, PA_DEV_BAD_SLOT, PA_ERR_HIP, PA_ERR_INVALID, PA_ERR_NO_BLOCKS, PA_ERR_NOT_FOUND,
    PA_ERR_REFCOUNT, PA_ERR_UNSUPPORTED, PA_F32, PA_OK, Allocator, PAError, SplitFuse, pa_abi_version, pa_copy_blocks,
    pa_decode_step, pa_decode_step_stage, pa_decode_step_staging_bytes,
    pa_forward, pa_forward_noalloc, pa_forward_noalloc_max_workspace_bytes, pa_forward_shared, pa_forward_shared_workspace_bytes, pa_forward_workspace_bytes, pa_last_error, pa_reshape_and_cache, pa_rope_reshape_and_cache, pa_set_stage_events,
)
