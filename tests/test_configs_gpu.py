"""GPU parity at the five named workloads' full sizes, in the launch
configuration bench.py times.

Decode workloads are checked on every row. For the two extend workloads the
oracle computes sampled rows and blocks one by one; every row and block is
also checked against properties that hold at any size (padding count,
causality, distinct positions, union ordering and membership popcounts).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import Dev, check_attention, check_topk_rows_valid, i32, log, to_np, torch_mod
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_relu_amd as m

    m.load()
    return m


def _topk(dsa, d, bt, k, mql):
    torch = torch_mod()
    out = dsa.indexer_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens, bt["cu"],
                           k, mql)
    torch.cuda.synchronize()
    return out


_TOPK_MEMO = {}


def _oracle_rows_topk(wl, b, rows):
    """Oracle top-k of the given rows (the rest -1), memoised per workload
    and row set so that the two query-block sizes of one workload share it."""
    key = (wl.name, b.T, tuple(rows))
    if key not in _TOPK_MEMO:
        _TOPK_MEMO.clear()
        _TOPK_MEMO[key] = _oracle_rows_topk_uncached(wl, b, rows)
    return _TOPK_MEMO[key]


def _oracle_rows_topk_uncached(wl, b, rows):
    return oracle.indexer_topk(bf16_to_f64(b.q_idx), b.w.astype(np.float64),
                               wl.idx_cache.f64_view(), wl.page_table, wl.seq_lens, b.cu_q_lens,
                               wl.k, rows=rows)


def _oracle_rows_mla(wl, b, topk, rows, layer=0):
    return oracle.sparse_mla(bf16_to_f64(b.q_mla[layer]), wl.kv_cache[layer].f64_view(),
                             wl.page_table, wl.seq_lens, b.cu_q_lens, topk, wl.sm_scale, wl.Dv,
                             rows=rows)


def _sample_rows(T, cu, n_random, seed, seq_lens=None):
    """Rows for the one-by-one oracle comparison: the first and last rows of
    the batch and of every sequence, rows at which a row's valid length
    crosses a multiple of the 2048-position scorer tile and of the
    16384-position select chunk, and n_random further rows stratified over
    the eight row positions of a scorer tile (t mod 8)."""
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    for c in cu[1:-1]:
        rows.update({int(c) - 1, int(c)})
    if seq_lens is not None:
        for s in range(len(cu) - 1):
            q0, q1 = int(cu[s]), int(cu[s + 1])
            a0 = int(seq_lens[s]) - (q1 - q0)
            for step in (2048, 16384):
                # row t has n_valid = a0 + (t - q0) + 1 positions
                for m in range(((a0 + 1) // step + 1) * step, a0 + (q1 - q0) + 1, step):
                    t = q0 + (m - a0 - 1)
                    rows.update({t - 1, t})
    per = max(1, n_random // 8)
    for r8 in range(8):
        cand = np.arange(r8, T, 8)
        rows.update(rng.choice(cand, size=min(per, cand.size), replace=False).tolist())
    return sorted(r for r in rows if 0 <= r < T)


def _decode_config(dsa, cid):
    torch = torch_mod()
    log(f"config {cid}: generating")
    wl = W.config(cid)
    b = wl.batches["decode"]
    d = Dev(wl)
    bt = d.batch("decode")
    log(f"config {cid}: indexer top-k, T={b.T}")
    tk = _topk(dsa, d, bt, wl.k, 1).cpu().numpy()
    rows = list(range(b.T))
    exp = _oracle_rows_topk(wl, b, rows)
    assert np.array_equal(tk, exp), "top-k differs from the oracle"
    log(f"config {cid}: sparse MLA decode")
    out = dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"],
                                i32(tk, "cuda"), wl.sm_scale)
    torch.cuda.synchronize()
    check_attention(to_np(out), _oracle_rows_mla(wl, b, exp, rows), what=f"config {cid} decode")


def test_config2_decode_batch(dsa):
    _decode_config(dsa, 2)


def test_config2_page_level_decode(dsa):
    """Page-level selection at the decode-batch size (k / PS = 32 pages of
    64 positions): page top-k on every row, then attention over the pages."""
    torch = torch_mod()
    wl = W.config(2)
    b = wl.batches["decode"]
    d = Dev(wl)
    bt = d.batch("decode")
    kp = wl.k // wl.PS
    log(f"config 2: page top-k, k_pages={kp}")
    pages = dsa.indexer_page_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens,
                                  bt["cu"], kp, 1)
    tok = dsa.page_tokens(pages, wl.PS)
    torch.cuda.synchronize()
    exp = oracle.indexer_page_topk(bf16_to_f64(b.q_idx), b.w.astype(np.float64),
                                   wl.idx_cache.f64_view(), wl.page_table, wl.seq_lens,
                                   b.cu_q_lens, kp)
    assert np.array_equal(pages.cpu().numpy(), exp), "page top-k differs from the oracle"
    exp_tok = oracle.page_tokens(exp, wl.PS)
    assert np.array_equal(tok.cpu().numpy(), exp_tok)
    log("config 2: attention over the selected pages")
    out = dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"], tok,
                                wl.sm_scale)
    torch.cuda.synchronize()
    ref = _oracle_rows_mla(wl, b, exp_tok, list(range(b.T)))
    check_attention(to_np(out), ref, what="config 2 page-level decode")
    out = dsa.sparse_mla_decode_pages(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens,
                                      bt["cu"], pages, wl.sm_scale)
    torch.cuda.synchronize()
    check_attention(to_np(out), ref, what="config 2 page-level decode (page lists)")


@pytest.mark.timeout(600)
def test_config3_ragged_decode(dsa):
    _decode_config(dsa, 3)


@pytest.mark.timeout(600)
def test_config3_page_level_decode(dsa):
    """Page-level selection on the ragged decode (rows of 4K..32K positions,
    k / PS = 32 pages): page top-k of every row checked for its padding and
    range, eight sampled rows against the oracle, then the page-list
    attention of those rows."""
    torch = torch_mod()
    wl = W.config(3)
    b = wl.batches["decode"]
    d = Dev(wl)
    bt = d.batch("decode")
    kp = wl.k // wl.PS
    pages = dsa.indexer_page_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens,
                                  bt["cu"], kp, 1)
    out = dsa.sparse_mla_decode_pages(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens,
                                      bt["cu"], pages, wl.sm_scale)
    torch.cuda.synchronize()
    got = pages.cpu().numpy()
    npg = -(-wl.seq_lens // wl.PS)  # decode rows: every position of the sequence is valid
    assert ((got >= 0) == (np.arange(kp)[None, :] < np.minimum(kp, npg)[:, None])).all()
    assert (got < npg[:, None]).all()
    rows = sorted({0, b.T - 1} | set(np.random.default_rng(3).choice(b.T, 6, replace=False).tolist()))
    log(f"config 3: page top-k oracle on rows {rows}")
    exp = oracle.indexer_page_topk(bf16_to_f64(b.q_idx), b.w.astype(np.float64),
                                   wl.idx_cache.f64_view(), wl.page_table, wl.seq_lens,
                                   b.cu_q_lens, kp, rows=rows)
    assert np.array_equal(got[rows], exp[rows]), "page top-k differs from the oracle"
    ref = _oracle_rows_mla(wl, b, oracle.page_tokens(exp, wl.PS), rows)
    check_attention(to_np(out), ref, rows=rows, what="config 3 page-level decode")


def _check_union_all_blocks(units, counts, member, topk, QB, u_max):
    """Properties of every block: sorted unique units, -1 tail, and per query
    popcount = number of selections (lossless caps)."""
    nqb = units.shape[0]
    T = topk.shape[0]
    assert (counts <= u_max).all(), "a block overflowed a lossless cap"
    for b in range(nqb):
        n = int(counts[b])
        assert (np.diff(units[b, :n]) > 0).all() and (units[b, n:] == -1).all()
    bytes_ = member.view(np.uint8).reshape(nqb, u_max, QB, 8)
    table = np.array([bin(i).count("1") for i in range(256)], dtype=np.uint8)
    pop = table[bytes_].sum(axis=(1, 3), dtype=np.int64)  # [nQB, QB]
    sel = np.zeros(nqb * QB, dtype=np.int64)
    sel[:T] = (topk >= 0).sum(axis=1)
    assert np.array_equal(pop.reshape(-1), sel), "membership popcount != selections"


def _extend_config(dsa, cid, QB, n_random, n_blocks):
    torch = torch_mod()
    log(f"config {cid}: generating")
    wl = W.config(cid)
    b = wl.batches["extend"]
    cu = b.cu_q_lens
    d = Dev(wl)
    bt = d.batch("extend")
    T = b.T
    mql = int(np.diff(cu).max())
    log(f"config {cid}: indexer top-k (tile path), T={T}")
    tk_t = _topk(dsa, d, bt, wl.k, mql)
    tk = tk_t.cpu().numpy()
    check_topk_rows_valid(tk, wl.seq_lens, cu, wl.k)
    rows = _sample_rows(T, cu, n_random, cid, wl.seq_lens)
    log(f"config {cid}: oracle top-k on {len(rows)} rows")
    exp = _oracle_rows_topk(wl, b, rows)
    assert np.array_equal(tk[rows], exp[rows]), "top-k differs from the oracle"
    # the same selection in position order (the attention's feed in the
    # layer loop): every row equals the canonical row sorted by position
    tk_pos = dsa.indexer_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens,
                              bt["cu"], wl.k, mql, order="position")
    torch.cuda.synchronize()
    big = np.iinfo(np.int64).max
    srt = np.sort(np.where(tk >= 0, tk.astype(np.int64), big), axis=1)
    assert np.array_equal(tk_pos.cpu().numpy(), np.where(srt == big, -1, srt)), \
        "position-order top-k is not the canonical selection sorted"

    log(f"config {cid}: union QB={QB}")
    u_max = wl.u_max
    units, counts, member = dsa.block_union(tk_t, d.seq_lens, bt["cu"], wl.PS, wl.MP, QB, u_max)
    torch.cuda.synchronize()
    un, cn, mn = units.cpu().numpy(), counts.cpu().numpy(), member.cpu().numpy()
    _check_union_all_blocks(un, cn, mn, tk, QB, u_max)
    nqb = un.shape[0]
    blocks = sorted({0, nqb - 1} | set(np.random.default_rng(cid).choice(
        nqb, min(n_blocks, nqb), replace=False).tolist()))
    eu, ec, em = oracle.block_union(tk, wl.seq_lens, cu, wl.PS, wl.MP, QB, u_max, blocks=blocks)
    for blk in blocks:
        assert np.array_equal(un[blk], eu[blk]) and cn[blk] == ec[blk]
        assert np.array_equal(mn[blk], em[blk])
    log(f"config {cid}: union sizes min/mean/max {cn.min()}/{cn.mean():.1f}/{cn.max()}")

    for layer in range(len(wl.kv_cache)):
        log(f"config {cid}: extend attend layer {layer} (indexer selection)")
        out = dsa.sparse_mla_extend(bt["q"] if layer == 0 else d.batch("extend", layer)["q"],
                                    d.kv_cache[layer], d.page_table, d.seq_lens, bt["cu"], units,
                                    counts, member, QB, wl.sm_scale)
        torch.cuda.synchronize()
        got = to_np(out)
        ref = _oracle_rows_mla(wl, b, tk, rows, layer=layer)
        check_attention(got, ref, rows=rows, what=f"config {cid} QB={QB} layer {layer}")

    if QB == 256:
        # per-query attend of the same packed batch: every row gathers its own
        # selected rows (the decode kernels), no union
        log(f"config {cid}: per-query attend (indexer selection)")
        out = dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"],
                                    tk_t, wl.sm_scale)
        torch.cuda.synchronize()
        ref = _oracle_rows_mla(wl, b, tk, rows)
        check_attention(to_np(out), ref, rows=rows, what=f"config {cid} per-query")

    log(f"config {cid}: extend attend with the locality selection")
    loc = W.locality_selection(wl.seq_lens, cu, wl.k, 100 + cid)
    lt = i32(loc, "cuda")
    u2, c2, m2 = dsa.block_union(lt, d.seq_lens, bt["cu"], wl.PS, wl.MP, QB, u_max)
    out = dsa.sparse_mla_extend(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"], u2,
                                c2, m2, QB, wl.sm_scale)
    torch.cuda.synchronize()
    ref = _oracle_rows_mla(wl, b, loc, rows)
    check_attention(to_np(out), ref, rows=rows, what=f"config {cid} QB={QB} locality")


@pytest.mark.timeout(600)
def test_config4_fused_indexer_every_row(dsa):
    """The chunked extend's indexer through the fused path (scores never
    stored; one segment per row at T = 4096) equals the score-matrix path
    on every row, and the oracle on the sampled rows."""
    torch = torch_mod()
    wl = W.config(4, with_mla=False)
    b = wl.batches["extend"]
    cu = b.cu_q_lens
    d = Dev(wl, layers=0)
    bt = d.batch("extend")
    mql = int(np.diff(cu).max())
    log("config 4: indexer top-k, score-matrix path and fused path")
    tk = _topk(dsa, d, bt, wl.k, mql).cpu().numpy()
    tf = dsa.indexer_topk_fused(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens,
                                bt["cu"], wl.k)
    torch.cuda.synchronize()
    tf = tf.cpu().numpy()
    assert np.array_equal(tf, tk), "fused and score-matrix top-k differ"
    rows = _sample_rows(b.T, cu, 64, 44, wl.seq_lens)
    exp = _oracle_rows_topk(wl, b, rows)
    assert np.array_equal(tf[rows], exp[rows]), "fused top-k differs from the oracle"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("QB", [64, 256])
def test_config4_chunked_extend(dsa, QB):
    _extend_config(dsa, 4, QB, n_random=256, n_blocks=8)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("QB", [256, 64])
def test_config5_long_indexshare(dsa, QB):
    _extend_config(dsa, 5, QB, n_random=128, n_blocks=8)


def test_config1_tiny_all_paths(dsa):
    """Tiny workload at its stated sizes: both indexer kernels, both QB."""
    torch = torch_mod()
    wl = W.config(1)
    d = Dev(wl)
    for bname in ("decode", "extend"):
        b = wl.batches[bname]
        bt = d.batch(bname)
        exp = _oracle_rows_topk(wl, b, list(range(b.T)))
        for mql in (1, 32):
            assert np.array_equal(_topk(dsa, d, bt, wl.k, mql).cpu().numpy(), exp)
    b = wl.batches["extend"]
    bt = d.batch("extend")
    tk = _oracle_rows_topk(wl, b, list(range(b.T)))
    ref = _oracle_rows_mla(wl, b, tk, list(range(b.T)))
    for QB in wl.QB:
        u, c, m = dsa.block_union(i32(tk, "cuda"), d.seq_lens, bt["cu"], wl.PS, wl.MP, QB,
                                  wl.u_max)
        out = dsa.sparse_mla_extend(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"],
                                    u, c, m, QB, wl.sm_scale)
        torch.cuda.synchronize()
        check_attention(to_np(out), ref, what=f"tiny QB={QB}")
