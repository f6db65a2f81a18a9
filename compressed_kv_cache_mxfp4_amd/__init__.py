"""MI355X (gfx950) implementation of the CSA2 decode hot path over an FP4
global KV cache: cache write, hierarchical sparse indexer (Full and Reindex
modes) and sparse attention, as hand-written HIP kernels behind the C ABI in
include/csa2.h.  This package is the thin Python binding (ctypes + torch for
device memory and streams)."""
from ._lib import (  # noqa: F401
    E4M3,
    E8M0,
    SWA_FP8,
    SWA_MAIN,
    Csa2Error,
    append_state,
    cache_append,
    cache_append_paged,
    cache_write,
    index_full,
    index_full_score,
    index_full_select,
    index_full_mq,
    index_full_paged,
    index_pool_rows,
    paged_alloc,
    index_pool,
    index_pool_mq,
    index_pool_score,
    index_pool_select,
    lib,
    quantize_fp4,
    sparse_attn_decode,
    sparse_attn_decode_mq,
    sparse_attn_decode_noalloc,
    sparse_attn_decode_rows,
    window_alloc,
    window_write,
    workspace,
)

MAIN_DIM = 512
IDX_DIM = 128
TOPK = 512
BLOCK = 8
POOL_BLOCKS = 2048
SWA = 128
ATTN_HEADS = 64
