"""Hybrid sliding-window / full GQA attention over a dual-pool KV cache,
for AMD Instinct MI355X (gfx950).

The compute path is libhybridattn.so (hand-written HIP kernels behind a C
ABI, include/hybrid_attn.h); this package is its Python binding plus the
host-side pool bookkeeping (pool tensors, page free list) and the 6:1 layer
group step plans. Importing the package does not load the library; the first
call does, and fails loudly if it has not been built.
"""

from ._lib import HA_BF16, HA_F32, HA_FULL, HA_KV_BF16, HA_KV_INT8, HA_SWA, HybridAttnError  # noqa: F401
from .api import (  # noqa: F401
    FullPagePool,
    HeadShape,
    KvView,
    PageAllocator,
    SwaRingPool,
    full_pool_append,
    full_pool_read,
    hybrid_attn_decode,
    hybrid_attn_decode_noalloc,
    hybrid_attn_decode_splits,
    hybrid_attn_prefill,
    hybrid_attn_verify,
    hybrid_attn_verify_workspace_size,
    hybrid_attn_workspace_size,
    swa_ring_append,
    swa_ring_read,
    window_safe_match,
)
