"""DeepSeek-Sparse-Attention hot path for MI355X (gfx950).

Python face of ``libdsa.so`` (C ABI in ``include/dsa.h``): exact
lightning-indexer top-k, query-block union tables, and sparse absorbed-MLA
attention for decode and chunked-prefill extend. All compute runs in the HIP
kernels; this package only marshals torch tensors into the C calls.
"""
from ._lib import (  # noqa: F401
    DSA_ORDER_POSITION,
    DSA_ORDER_SCORE,
    DsaError,
    block_union,
    block_union_workspace,
    extend_attend_path,
    extend_attend_plan,
    extend_layers,
    header_functions,
    index_share_map,
    indexer_page_topk,
    indexer_page_topk_workspace,
    indexer_topk,
    indexer_topk_fused,
    indexer_topk_fused_workspace,
    indexer_topk_workspace,
    last_error,
    load,
    page_tokens,
    paged_write,
    paged_write_layer,
    profile_enable,
    profile_read,
    sparse_mla_decode,
    sparse_mla_decode_pages,
    sparse_mla_decode_static,
    sparse_mla_decode_workspace,
    sparse_mla_extend,
    sparse_mla_extend_workspace,
    status_string,
    topk_position_order,
)
