"""Paged-attention decode for AMD MI355X (gfx950): Python face of libpagedattn.

The compute runs in hand-written HIP kernels behind a C ABI
(``include/pagedattn.h``); this package only marshals torch tensors into it.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    NOALLOC_SCRATCH_BYTES,
    PA_BF16,
    PA_F32,
    BlockManager,
    DecodeLaunch,
    PagedAttnError,
    PoolExhausted,
    declared_functions,
    kv_append,
    kv_append_layers,
    kv_append_tokens,
    kv_cow_copy,
    kv_swap_in,
    kv_swap_out,
    load,
    make_dims,
    paged_attn_decode,
    paged_attn_decode_append,
    paged_attn_decode_noalloc,
    paged_attn_extend,
    paged_attn_extend_plan,
    paged_attn_order,
    paged_attn_plan,
    paged_attn_workspace_bytes,
    paged_kv_gather,
)
