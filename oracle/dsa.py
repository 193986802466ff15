"""CPU oracle for the DeepSeek-Sparse-Attention hot path (fp64, NumPy).

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously
correct statement of what the GPU library must compute. Only the tests,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it; the GPU product path never calls it and shares no code with it.

Sources (the sglang-jax DSA pages; every citation names the page and the
function on it):

* "ref.py" page, ``streamindex_topk_ref``: the lightning-indexer score
  ``sum_h w_h * relu(q_h . k)``, the causal mask ``j <= abs_q`` with
  ``abs_q = kv_len - q_len + (t - q_start)``, the ``j < kv_len`` mask and
  the -1 padding rule (a slot is real only when its rank is below the
  number of valid positions and its score is finite).
* "ref.py" page, ``sparse_mla_ref``: sparse absorbed MLA, logits over the
  full packed ``[nope | rope]`` row times ``sm_scale``, masked softmax,
  value = the first ``v_dim`` columns of the same latent row, an empty
  selection gives zeros.
* "sparse_mla_prefill_qblock.py" page, ``build_block_unit_tables``: the
  per-query-block sorted unique union of selected units, its true
  (uncapped) size, truncation to ``u_max`` slots and membership by slot;
  and ``sparse_mla_attention_qblock`` (ragged mode): seq-local units lifted
  to global keys by the request's page-table base, blocks packed over the
  ragged token axis and allowed to straddle requests.

* "ref.py" page, ``streamindex_page_topk_ref``: the page-level indexer,
  token scores max-pooled per page and the top ``k_pages`` pages.
* "dsa_sparse_backend.py" page, ``_scatter_paged``, and
  "sparse_mla_prefill_qblock.py" page, ``paged_write_back``: the paged
  cache self-write of the new tokens ahead of the attention.

Readings taken where the pages leave a step open (each is a row of the
design notes' list of readings):

* top-k is exact (the pages' approximate first stage is not reproducible);
  order is score descending, then position ascending; ties go to the lower
  position; -0.0 equals +0.0;
* positions are seq-local token indices; the page table has a fixed stride
  ``MP`` per sequence; a page unit's global key is ``s * MP + j // PS``;
* membership is per token: bit ``j % PS`` of a 64-bit word per (slot, query),
  because the selection is token-exact;
* the attention applies both ``j < kv_len`` (``sparse_mla_ref``) and the
  causal bound ``j <= abs_q`` (the qblock kernel's ``kp <= qpos``).

Parity pins: see ``tests/test_oracle.py`` (brute force, closed forms,
hand-worked fixtures, invariants and planted-mistake checks).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------
# Ragged bookkeeping
# ----------------------------------------------------------------------------
def query_rows(seq_lens, cu_q_lens, T):
    """Per packed row t: (sequence id or -1, absolute position or -1).

    "ref.py" page, ``streamindex_topk_ref`` general path:
    ``abs_q = kv_len - (q_end - q_start) + (t - q_start)`` for rows with
    ``q_start <= t < q_end``; rows in no sequence belong to none.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    seq = np.full(T, -1, dtype=np.int64)
    pos = np.full(T, -1, dtype=np.int64)
    for s in range(len(seq_lens)):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        for t in range(q0, min(q1, T)):
            seq[t] = s
            pos[t] = int(seq_lens[s]) - (q1 - q0) + (t - q0)
    return seq, pos


def n_valid_keys(kv_len, abs_q):
    """Number of positions j with j < kv_len and j <= abs_q ("ref.py",
    ``streamindex_topk_ref`` mask)."""
    return int(max(0, min(int(kv_len), int(abs_q) + 1)))


def gather_rows(cache, page_table, s, positions):
    """Rows of a paged cache for seq-local positions of sequence ``s``.

    Position j of sequence s lives in physical page ``page_table[s, j // PS]``
    at offset ``j % PS`` ("ref.py" page: ``cache_kv[seq_pages]`` reshaped to
    ``[max_kv, D]``; fixed-stride table as produced by the backend page's
    ``_fixed_stride_pages``).
    """
    PS = cache.shape[1]
    positions = np.asarray(positions, dtype=np.int64)
    pages = page_table[s, positions // PS]
    return cache[pages, positions % PS]


# ----------------------------------------------------------------------------
# Lightning indexer
# ----------------------------------------------------------------------------
def head_mix(dots, w):
    """``sum_h w_h * relu(dots[:, h])`` ("ref.py", ``streamindex_topk_ref``:
    ReLU on each head's dot, then the weighted head sum)."""
    return np.maximum(dots, 0.0) @ w


def indexer_scores(q_t, w_t, keys):
    """fp64 scores of one query row against keys [n, D].

    q_t [H, D], w_t [H]; ``dots[j, h] = q_t[h] . keys[j]``.
    """
    dots = keys @ q_t.T
    return head_mix(dots, w_t)


def canonical_order(scores):
    """Indices sorted by score descending, ties by lower position first.

    A full sort (``numpy.lexsort``); the pages' two-stage approximate top-k
    is replaced by the exact order. Comparison treats -0.0 == +0.0.
    """
    n = scores.shape[0]
    return np.lexsort((np.arange(n), -scores))


def indexer_topk(q, w, idx_cache, page_table, seq_lens, cu_q_lens, k, rows=None):
    """Exact token top-k of the lightning indexer.

    "ref.py" page, ``streamindex_topk_ref`` (general causal path; decode is
    the case q_len == 1, where the causal bound equals ``kv_len - 1``):
    for row t of sequence s at absolute position a, score every j with
    j < kv_len and j <= a, keep the first min(k, n_valid) positions of the
    canonical order, pad with -1. Rows outside every sequence stay -1.

    q [T, H, D] float64, w [T, H], idx_cache [P, PS, D], page_table [S, MP],
    returns int32 [T, k]. ``rows`` restricts the work to some rows (others
    are left -1).
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T = q.shape[0]
    seq, pos = query_rows(seq_lens, cu_q_lens, T)
    out = np.full((T, k), -1, dtype=np.int32)
    for t in range(T) if rows is None else rows:
        s = int(seq[t])
        if s < 0:
            continue
        n = n_valid_keys(seq_lens[s], pos[t])
        if n == 0:
            continue
        keys = np.asarray(gather_rows(idx_cache, page_table, s, np.arange(n)), dtype=np.float64)
        scores = indexer_scores(q[t], w[t], keys)
        order = canonical_order(scores)[: min(k, n)]
        out[t, : order.size] = order
    return out


def indexer_score_row(q, w, idx_cache, page_table, seq_lens, cu_q_lens, t):
    """All valid scores of row t (fp64), for diagnostics and tests."""
    T = q.shape[0]
    seq, pos = query_rows(seq_lens, cu_q_lens, T)
    s = int(seq[t])
    if s < 0:
        return np.zeros(0)
    n = n_valid_keys(seq_lens[s], pos[t])
    keys = np.asarray(gather_rows(idx_cache, page_table, s, np.arange(n)), dtype=np.float64)
    return indexer_scores(np.asarray(q[t], np.float64), np.asarray(w[t], np.float64), keys)


def page_pool(scores, PS):
    """Page scores of a row whose valid positions are 0 .. n-1: page p is the
    maximum over its valid positions p*PS .. min((p+1)*PS, n) - 1 ("ref.py",
    ``streamindex_page_topk_ref``: masked positions at -inf, then a max over
    the page axis). Only pages holding a valid position are returned."""
    n = scores.shape[0]
    n_pages = -(-n // PS)
    padded = np.full(n_pages * PS, -np.inf)
    padded[:n] = scores
    return padded.reshape(n_pages, PS).max(axis=1)


def indexer_page_topk(q, w, idx_cache, page_table, seq_lens, cu_q_lens, k_pages, rows=None):
    """Exact page-level top-k of the lightning indexer.

    "ref.py" page, ``streamindex_page_topk_ref``: the token scores of
    ``streamindex_topk_ref`` with every masked position (j >= kv_len or
    j > abs_q) at -inf, max-pooled over the PS positions of each seq-local
    page; the top ``k_pages`` pages of that page score, -1 where the score is
    -inf (a page with no valid position) and past the last page.

    Read exactly (like the token top-k): pages in the canonical order, page
    score descending, ties to the lower page id. A page is valid iff it holds
    a valid position, i.e. the first ceil(n_valid / PS) pages of the row.

    Returns int32 [T, k_pages] of seq-local page ids.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    PS = idx_cache.shape[1]
    T = q.shape[0]
    seq, pos = query_rows(seq_lens, cu_q_lens, T)
    out = np.full((T, k_pages), -1, dtype=np.int32)
    for t in range(T) if rows is None else rows:
        s = int(seq[t])
        if s < 0:
            continue
        n = n_valid_keys(seq_lens[s], pos[t])
        if n == 0:
            continue
        keys = np.asarray(gather_rows(idx_cache, page_table, s, np.arange(n)), dtype=np.float64)
        page_scores = page_pool(indexer_scores(q[t], w[t], keys), PS)
        order = canonical_order(page_scores)[: min(k_pages, page_scores.size)]
        out[t, : order.size] = order
    return out


def page_tokens(pages, PS):
    """Positions of the selected pages: row t lists, for each slot i of
    ``pages[t]``, the positions ``pages[t, i] * PS + r`` for r < PS (-1 for
    a -1 slot). The attention over them masks j >= kv_len and j > abs_q
    itself, so a page that runs past the sequence end only contributes its
    valid positions ("ref.py", ``sparse_mla_ref`` masks; the page-budget
    decode of the backend page attends all valid tokens of its pages)."""
    pages = np.asarray(pages, dtype=np.int64)
    T, kp = pages.shape
    r = np.arange(PS, dtype=np.int64)
    tok = pages[:, :, None] * PS + r[None, None, :]
    tok = np.where(pages[:, :, None] >= 0, tok, -1)
    return tok.reshape(T, kp * PS).astype(np.int32)


# ----------------------------------------------------------------------------
# Paged cache writes
# ----------------------------------------------------------------------------
def paged_write(cache, rows, col0, page_table, seq_lens, cu_q_lens):
    """The cache after the new rows are written ("dsa_sparse_backend.py",
    ``_scatter_paged``; "sparse_mla_prefill_qblock.py", ``paged_write_back``):
    packed row t of sequence s goes to seq-local position
    ``a = seq_lens[s] - q_len(s) + (t - q_start)``, i.e. physical page
    ``page_table[s, a // PS]`` at offset ``a % PS``, columns
    ``col0 .. col0 + cols - 1``; the other columns and slots are unchanged.

    Reading taken: rows outside every sequence, positions outside
    ``0 <= a < min(seq_lens[s], MP * PS)``, and positions whose page-table
    entry is not a page of the cache (outside ``[0, P)``, e.g. -1 for an
    unassigned page) have no slot and are dropped (the pages route such rows
    to a reserved page of their allocator instead).

    cache [P, PS, C], rows [T, cols]; returns a new array.
    """
    out = np.array(cache, copy=True)
    rows = np.asarray(rows)
    T, cols = rows.shape
    P, PS = cache.shape[0], cache.shape[1]
    MP = page_table.shape[1]
    seq, pos = query_rows(seq_lens, cu_q_lens, T)
    for t in range(T):
        s, a = int(seq[t]), int(pos[t])
        if s < 0 or a < 0 or a >= min(int(seq_lens[s]), MP * PS):
            continue
        page = int(page_table[s, a // PS])
        if page < 0 or page >= P:
            continue
        out[page, a % PS, col0:col0 + cols] = rows[t]
    return out


# ----------------------------------------------------------------------------
# Query-block union and membership
# ----------------------------------------------------------------------------
def unit_key(s, j, MP, PS):
    """Global page key of seq-local position j of sequence s.

    "sparse_mla_prefill_qblock.py" page, ``sparse_mla_attention_qblock``
    ragged mode lifts a seq-local page to ``base_page + page``; with a
    fixed-stride table the base of sequence s is ``s * MP``.
    """
    return int(s) * MP + int(j) // PS


def member_bit(j, PS):
    """Bit of position j inside its page's 64-bit membership word."""
    return 1 << (int(j) % PS)


def block_union(topk, seq_lens, cu_q_lens, PS, MP, QB, u_max, blocks=None):
    """Per query-block union tables.

    "sparse_mla_prefill_qblock.py" page, ``build_block_unit_tables``: pad
    the packed rows to a multiple of QB with empty rows, take the sorted set
    of selected unit keys per block (-1 entries ignored), report its true
    size uncapped, keep the first ``u_max`` keys (-1 padded), and give each
    (slot, query) pair its membership; here the membership is the OR of
    ``1 << (j % PS)`` over the query's selected positions j in that page.

    Entries j < 0 and j >= MP * PS (no page-table column) are ignored, and
    rows outside every sequence contribute nothing.

    Returns (units int32 [nQB, u_max], counts int32 [nQB],
    member uint64 [nQB, u_max, QB]). ``blocks`` restricts the work to some
    blocks (the others are left empty).
    """
    topk = np.asarray(topk)
    T = topk.shape[0]
    seq, _ = query_rows(seq_lens, cu_q_lens, T)
    nqb = -(-T // QB)
    units = np.full((nqb, u_max), -1, dtype=np.int32)
    counts = np.zeros(nqb, dtype=np.int32)
    member = np.zeros((nqb, u_max, QB), dtype=np.uint64)
    for b in range(nqb) if blocks is None else blocks:
        picks = []  # (query-in-block, key, bit)
        for qi in range(QB):
            t = b * QB + qi
            if t >= T or seq[t] < 0:
                continue
            for j in topk[t]:
                j = int(j)
                if j < 0 or j >= MP * PS:
                    continue
                picks.append((qi, unit_key(seq[t], j, MP, PS), member_bit(j, PS)))
        keys = sorted({key for _, key, _ in picks})
        counts[b] = len(keys)
        kept = keys[:u_max]
        units[b, : len(kept)] = kept
        slot = {key: i for i, key in enumerate(kept)}
        for qi, key, bit in picks:
            if key in slot:
                member[b, slot[key], qi] |= np.uint64(bit)
    return units, counts, member


# ----------------------------------------------------------------------------
# Sparse absorbed MLA
# ----------------------------------------------------------------------------
def valid_selection(sel, kv_len, abs_q):
    """Selected positions that take part in attention: j >= 0, j < kv_len
    ("ref.py", ``sparse_mla_ref``) and j <= abs_q (the qblock kernel's
    causal term). Order and multiplicity are kept as given."""
    sel = np.asarray(sel, dtype=np.int64)
    return sel[(sel >= 0) & (sel < kv_len) & (sel <= abs_q)]


def softmax(logits):
    """Row softmax with the row maximum subtracted."""
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=-1, keepdims=True)


def attend(q_t, rows, sm_scale, v_dim):
    """One query's heads over gathered latent rows.

    q_t [H, Dk], rows [n, Dk]: logits = sm_scale * q_t @ rows.T over the
    whole packed row ("ref.py", ``sparse_mla_ref``), softmax over the n
    rows, output = p @ rows[:, :v_dim].
    """
    logits = sm_scale * (q_t @ rows.T)
    p = softmax(logits)
    return p @ rows[:, :v_dim]


def sparse_mla(q, kv_cache, page_table, seq_lens, cu_q_lens, topk, sm_scale, v_dim=512,
               rows=None):
    """Sparse absorbed-MLA attention over each query's own selection.

    "ref.py" page, ``sparse_mla_ref`` (both decode and extend use this
    definition; the qblock kernel's page is stated to match its semantics):
    q [T, H, Dk] float64 packed ``[nope | rope]``, kv_cache [P, PS, >=Dk]
    packed ``[c_kv | k_rope]``, topk [T, k] seq-local positions (-1 = none).
    A row with no valid selection, or outside every sequence, is 0.
    Returns float64 [T, H, v_dim].
    """
    q = np.asarray(q, dtype=np.float64)
    T, H, Dk = q.shape
    seq, pos = query_rows(seq_lens, cu_q_lens, T)
    out = np.zeros((T, H, v_dim), dtype=np.float64)
    for t in range(T) if rows is None else rows:
        s = int(seq[t])
        if s < 0:
            continue
        sel = valid_selection(topk[t], seq_lens[s], pos[t])
        if sel.size == 0:
            continue
        kv = np.asarray(gather_rows(kv_cache, page_table, s, sel), dtype=np.float64)[:, :Dk]
        out[t] = attend(q[t], kv, sm_scale, v_dim)
    return out
