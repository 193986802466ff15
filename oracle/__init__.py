"""CPU oracle for the DeepSeek-Sparse-Attention hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the GPU library. It is an
independent fp64 NumPy statement of the method and shares no code with the
HIP kernels.
"""
from .dsa import (  # noqa: F401
    attend,
    block_union,
    canonical_order,
    gather_rows,
    head_mix,
    indexer_score_row,
    indexer_scores,
    indexer_page_topk,
    indexer_topk,
    page_tokens,
    paged_write,
    member_bit,
    n_valid_keys,
    query_rows,
    softmax,
    sparse_mla,
    unit_key,
    valid_selection,
)
