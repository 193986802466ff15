"""GPU parity: every entry point of libdsa.so against the fp64 oracle.

Top-k and union tables are compared bit for bit (the indexer inputs are
integer-valued, so fp32 scores are exact in any summation order); attention
outputs within max-abs 2e-2 and relative-L2 5e-3. Shapes here are small
enough for the oracle to finish in seconds while spanning several tiles,
ragged tails and the degenerate cases.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (Dev, bf16, check_attention, check_topk_rows_valid, f32, i32, log,
                         to_np, torch_mod)
from workloads import bf16_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_relu_amd as m

    m.load()  # fails loudly when the library is missing
    return m


def _oracle_topk(wl, b, k=None, q_idx=None, w=None, cu=None):
    q_idx = b.q_idx if q_idx is None else q_idx
    w = b.w if w is None else w
    cu = b.cu_q_lens if cu is None else cu
    return oracle.indexer_topk(bf16_to_f64(q_idx), w.astype(np.float64),
                               bf16_to_f64(wl.idx_cache), wl.page_table, wl.seq_lens, cu,
                               wl.k if k is None else k)


def _gpu_topk(dsa, d, q_idx, w, cu, k, max_q_len, order="score"):
    """max_q_len "fused" calls the fused entry point (scores never stored)."""
    torch = torch_mod()
    if max_q_len == "fused":
        out = dsa.indexer_topk_fused(bf16(q_idx, "cuda"), f32(w, "cuda"), d.idx_cache,
                                     d.page_table, d.seq_lens, i32(cu, "cuda"), k, order=order)
    else:
        out = dsa.indexer_topk(bf16(q_idx, "cuda"), f32(w, "cuda"), d.idx_cache, d.page_table,
                               d.seq_lens, i32(cu, "cuda"), k, max_q_len, order=order)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _by_position(topk):
    """Each row's non-negative entries ascending, then -1 (the position
    order of a top-k table)."""
    big = np.iinfo(np.int64).max
    t = np.where(topk >= 0, topk.astype(np.int64), big)
    t = np.sort(t, axis=1)
    return np.where(t == big, -1, t).astype(np.int32)


def _mql(path, ql):
    return 1 if path == "rows" else ("fused" if path == "fused" else max(2, ql))


def _max_q_len(cu):
    cu = np.asarray(cu)
    return int(np.diff(cu).max(initial=0))


# ----------------------------------------------------------------------------
# Indexer
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("bname", ["decode", "extend"])
@pytest.mark.parametrize("path", ["rows", "tiles", "fused"])
def test_indexer_tiny(dsa, bname, path):
    wl = W.config(1)
    b = wl.batches[bname]
    log(f"indexer tiny {bname} path={path}")
    d = Dev(wl)
    mql = _mql(path, _max_q_len(b.cu_q_lens))
    got = _gpu_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, wl.k, mql)
    exp = _oracle_topk(wl, b)
    assert np.array_equal(got, exp)
    got_p = _gpu_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, wl.k, mql, order="position")
    assert np.array_equal(got_p, _by_position(exp))


INDEXER_EDGE = {
    # name: (S, kv_lens, PS, MP, q_lens, H, D, k, extra_rows)
    "mixed_empty_seq_tail_rows": (3, [37, 200, 64], 16, 16, [1, 5, 0], 4, 32, 48, 3),
    "h64_d128_ragged": (2, [1000, 4097], 64, 80, [40, 33], 64, 128, 256, 0),
    "h1_d64_k1": (2, [77, 300], 32, 10, [3, 70], 1, 64, 1, 1),
    "k4096_short_rows": (2, [100, 2500], 64, 40, [1, 2], 32, 128, 4096, 0),
    "k4096_long_rows": (1, [10000], 64, 160, [3], 32, 128, 4096, 0),
    "h32_d128_chunk_straddle": (4, [700, 64, 1500, 33], 64, 24, [33, 64, 47, 33], 32, 128, 128, 2),
    # rows above 16384 positions (the select's key range then comes from the
    # tile scorer's per-2048-position extremes) sharing 8-row tiles with short
    # rows; 18433 positions leave a last tile of one position
    "h32_d128_long_rows_tile_extremes": (3, [40000, 300, 18433], 64, 640, [5, 2, 4], 32, 128,
                                         512, 1),
    # rows of several select chunks at the other list capacities (k up to
    # 1024, and k above 2048 where the candidate list is the shortest
    # relative to k)
    "h32_d128_long_rows_k1000": (2, [40000, 20000], 64, 640, [3, 2], 32, 128, 1000, 0),
    "h32_d128_long_rows_k4096": (2, [40000, 33000], 64, 640, [3, 2], 32, 128, 4096, 0),
    # score rows of two select chunks held in registers (workspace rows of
    # 32768 positions): rows of exactly one chunk, one position past it, and
    # the last positions of the second chunk
    "h32_d128_two_chunk_rows": (4, [16384, 16385, 32767, 32768], 64, 512, [1, 2, 1, 2], 32,
                                128, 2048, 0),
}


@pytest.mark.parametrize("name", sorted(INDEXER_EDGE))
@pytest.mark.parametrize("path", ["rows", "tiles", "fused"])
def test_indexer_edges(dsa, name, path):
    S, kv, PS, MP, ql, H, D, k, extra = INDEXER_EDGE[name]
    cu = np.concatenate([[0], np.cumsum(ql)]).tolist()
    wl = W.build(name=name, seed=77, S=S, kv_lens=kv, PS=PS, MP=MP, batches={"b": cu}, H_idx=H,
                 D_idx=D, k=k, with_mla=False, extra_pages=2)
    b = wl.batches["b"]
    q_idx, w = b.q_idx, b.w
    if extra:  # rows past cu_q_lens[S] belong to no sequence
        q_idx = np.concatenate([q_idx, q_idx[:1].repeat(extra, 0)])
        w = np.concatenate([w, w[:1].repeat(extra, 0)])
    log(f"indexer edge {name} path={path} T={q_idx.shape[0]}")
    d = Dev(wl)
    mql = _mql(path, max(ql))
    got = _gpu_topk(dsa, d, q_idx, w, cu, k, mql)
    exp = _oracle_topk(wl, b, k=k, q_idx=q_idx, w=w, cu=np.array(cu))
    assert np.array_equal(got, exp)
    check_topk_rows_valid(got, wl.seq_lens, cu, k)
    # the same set in position order (the fused path's lists, or a sort of
    # the selected rows after the score-matrix select)
    got_p = _gpu_topk(dsa, d, q_idx, w, cu, k, mql, order="position")
    assert np.array_equal(got_p, _by_position(exp))


@pytest.mark.parametrize("k", [1, 7, 256, 1000, 1024, 2048, 2049, 4096])
def test_topk_position_order_rows(dsa, k):
    """dsa_topk_position_order against a NumPy sort: rows with -1 entries
    anywhere, duplicates, position 0, large positions, all -1, in place and
    out of place."""
    torch = torch_mod()
    rng = np.random.default_rng(k)
    T = 37
    hi = [1, 5, 1 << 10, 1 << 17, (1 << 31) - 2]
    rows = []
    for t in range(T):
        v = rng.integers(0, hi[t % len(hi)], size=k, endpoint=True).astype(np.int64)
        v[rng.random(k) < (t % 4) / 4.0] = -1
        if t == 3:
            v[:] = -1
        rows.append(v)
    tk = np.stack(rows).astype(np.int32)
    log(f"top-k position order k={k}")
    src = i32(tk, "cuda")
    out = dsa.topk_position_order(src)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), _by_position(tk))
    dsa.topk_position_order(src, out=src)  # in place
    torch.cuda.synchronize()
    assert np.array_equal(src.cpu().numpy(), _by_position(tk))


# Ragged decode-style batches large enough (rows x 128-position stages above
# 2048) for the balanced scorers: rows of very different lengths, empty
# sequences, rows past the last sequence, H < 32, every D, page sizes that are
# and are not multiples of 32, and many short rows so that one wave's share
# spans many rows. Up to 1024 sequences take the register scorer (the last
# case: its limits, 1024 rows of 1024 sequences); 1100 sequences, half of
# them without rows, take the LDS-ring scorer.
INDEXER_FLAT = {
    # name: (S, kv range, q_len choices, PS, MP, H, D, k, extra_rows)
    "d128_h32_mixed": (40, (0, 4000), (0, 1, 1, 2, 5), 64, 64, 32, 128, 256, 3),
    "d64_h20_ps16": (100, (1, 3200), (1,), 16, 200, 20, 64, 100, 0),
    "d32_many_short_rows": (1000, (1, 300), (1,), 16, 160, 32, 32, 64, 2),
    "d128_ps48_h7": (40, (1, 6000), (1, 2), 48, 128, 7, 128, 300, 0),
    "d128_s1100_ring": (1100, (1, 400), (0, 1), 16, 32, 32, 128, 64, 0),
    "d64_ps32_max_rows": (1024, (1, 500), (1,), 32, 16, 32, 64, 64, 0),
}


@pytest.mark.parametrize("name", sorted(INDEXER_FLAT))
def test_indexer_flat(dsa, name):
    S, (lo, hi), qchoice, PS, MP, H, D, k, extra = INDEXER_FLAT[name]
    rng = np.random.default_rng(4242)
    ql = rng.choice(qchoice, size=S)
    kv = np.maximum(rng.integers(lo, hi + 1, size=S), ql)
    cu = np.concatenate([[0], np.cumsum(ql)]).tolist()
    wl = W.build(name=name, seed=78, S=S, kv_lens=kv.tolist(), PS=PS, MP=MP, batches={"b": cu},
                 H_idx=H, D_idx=D, k=k, with_mla=False, extra_pages=1)
    b = wl.batches["b"]
    q_idx, w = b.q_idx, b.w
    if extra:
        q_idx = np.concatenate([q_idx, q_idx[:1].repeat(extra, 0)])
        w = np.concatenate([w, w[:1].repeat(extra, 0)])
    T = q_idx.shape[0]
    assert T * -(-(MP * PS) // 128) > 2048
    log(f"indexer flat {name} T={T}")
    d = Dev(wl)
    got = _gpu_topk(dsa, d, q_idx, w, cu, k, 1)
    exp = _oracle_topk(wl, b, k=k, q_idx=q_idx, w=w, cu=np.array(cu))
    assert np.array_equal(got, exp)
    check_topk_rows_valid(got, wl.seq_lens, cu, k)


def test_indexer_ties_and_negative_zero(dsa):
    """All-zero queries (every score ties at 0) and negative weights (scores
    of -0.0 mixed with +0.0): order is by position."""
    wl = W.build(name="ties", seed=5, S=2, kv_lens=[300, 129], PS=16, MP=20,
                 batches={"b": [0, 4, 9]}, H_idx=8, D_idx=32, k=64, with_mla=False)
    b = wl.batches["b"]
    q = b.q_idx.copy()
    q[::2] = W.f32_to_bf16(np.zeros(q[::2].shape, np.float32))
    w = b.w.copy()
    w[1::2] *= -1.0
    d = Dev(wl)
    for mql in (1, 5, "fused"):
        log(f"indexer ties mql={mql}")
        got = _gpu_topk(dsa, d, q, w, b.cu_q_lens, 64, mql)
        exp = _oracle_topk(wl, b, k=64, q_idx=q, w=w)
        assert np.array_equal(got, exp)


@pytest.mark.parametrize("k,kv", [(200, 3000), (512, 3000), (512, 20000)])
def test_indexer_crowded_ties(dsa, k, kv):
    """All but 20 keys share one vector (exactly equal scores) and those 20
    are its double: the top-k is the 20 large scores, then the tied positions
    in ascending order. With k=200 the ties fill one bucket of the select's
    rank phase; with k=512 that bucket overflows and the list is sorted
    instead. At 20000 positions a row spans several select chunks and most
    2048-position tiles hold a single score value."""
    wl = W.build(name="crowded", seed=11, S=1, kv_lens=[kv], PS=64, MP=-(-kv // 64),
                 batches={"b": [0, 3]}, H_idx=8, D_idx=64, k=k, with_mla=False)
    b = wl.batches["b"]
    rows = wl.idx_cache.rows
    v = b.q_idx[0, 0].copy()
    rows[:] = v
    big = np.random.default_rng(3).choice(rows.shape[0], 20, replace=False)
    rows[big] = W.f32_to_bf16(2.0 * W.bf16_to_f32(v))
    d = Dev(wl)
    exp = _oracle_topk(wl, b, k=k)
    for mql in (1, 3, "fused"):
        log(f"indexer crowded ties k={k} kv={kv} mql={mql}")
        got = _gpu_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, k, mql)
        assert np.array_equal(got, exp)


@pytest.mark.parametrize("skew", ["early", "late"])
def test_indexer_long_rows_skewed(dsa, skew):
    """Rows of 40000 positions whose first 16384 keys (one select chunk) are
    doubled ("early": the top-k crowds into them) or whose later keys are
    ("late": far more large scores after the first chunk than it suggests).
    Doubling a key doubles every head's dot product, so the positions keep
    their order within each part; the select's estimate taken from the
    first chunk misses in both directions and the exact answer must hold."""
    kv = 40000
    wl = W.build(name="skewed", seed=21, S=1, kv_lens=[kv], PS=64, MP=-(-kv // 64),
                 batches={"b": [0, 3]}, H_idx=32, D_idx=128, k=2048, with_mla=False)
    b = wl.batches["b"]
    cache = wl.idx_cache
    pos = np.arange(16384) if skew == "early" else np.arange(16384, kv)
    phys = wl.page_table[0][pos // wl.PS].astype(np.int64) * wl.PS + pos % wl.PS
    at = np.searchsorted(cache.slots, phys)
    assert np.array_equal(cache.slots[at], phys)
    cache.rows[at] = W.f32_to_bf16(2.0 * W.bf16_to_f32(cache.rows[at]))
    d = Dev(wl)
    exp = _oracle_topk(wl, b, k=2048)
    for mql in (1, 3, "fused"):
        log(f"indexer long rows skew={skew} mql={mql}")
        got = _gpu_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, 2048, mql)
        assert np.array_equal(got, exp)
    check_topk_rows_valid(got, wl.seq_lens, b.cu_q_lens, 2048)


# The fused path: lists that fill and are cut many times per row (k small
# against the row length), scores rising with position (every key beats the
# bar, ties at every level), one score for every key (each cut is a tie cut
# by position), and few rows over a long context (several segments per row,
# merged).
FUSED_CASES = {
    # name: (S, kv_lens, PS, MP, q_lens, H, D, k, pattern)
    "k16_rows6000": (2, [6000, 4100], 16, 400, [9, 7], 8, 32, 16, "random"),
    "k100_rows_straddle": (3, [5000, 64, 9000], 64, 150, [5, 2, 11], 32, 128, 100, "random"),
    "rising_steps": (1, [9000], 64, 150, [10], 1, 32, 300, "rising"),
    "all_equal": (2, [7000, 3000], 32, 230, [6, 4], 4, 64, 257, "equal"),
    "segments_k2048": (2, [40000, 25000], 64, 640, [4, 3], 32, 128, 2048, "random"),
    "segments_k4096_h40": (1, [50000], 64, 800, [6], 40, 128, 4096, "random"),
    "k4096_one_segment": (2, [2000, 700], 64, 32, [5, 3], 32, 128, 4096, "random"),
}


@pytest.mark.parametrize("name", sorted(FUSED_CASES))
def test_indexer_fused_cases(dsa, name):
    S, kv, PS, MP, ql, H, D, k, pattern = FUSED_CASES[name]
    cu = np.concatenate([[0], np.cumsum(ql)]).tolist()
    wl = W.build(name=name, seed=91, S=S, kv_lens=kv, PS=PS, MP=MP, batches={"b": cu}, H_idx=H,
                 D_idx=D, k=k, with_mla=False, extra_pages=1)
    b = wl.batches["b"]
    q_idx, w = b.q_idx, b.w
    if pattern == "rising":
        # key at position j: its first m_j coordinates 2, the rest 0, with m_j
        # rising with j; queries all 2, one head of weight 1: score 4 m_j
        q_idx = W.f32_to_bf16(np.full(q_idx.shape, 2.0, np.float32))
        w = np.ones(w.shape, np.float32)
        n = wl.idx_cache.rows.shape[0]
        flat = wl.idx_cache.slots
        page_of = {int(p): i for i, p in enumerate(wl.page_table[0])}
        pos = np.array([page_of[int(sl) // PS] * PS + int(sl) % PS for sl in flat])
        m = np.minimum(D, pos * (D + 1) // kv[0])
        vals = (np.arange(D)[None, :] < m[:, None]).astype(np.float32) * 2.0
        wl.idx_cache.rows[:] = W.f32_to_bf16(vals)
        assert n == flat.size
    elif pattern == "equal":
        wl.idx_cache.rows[:] = wl.idx_cache.rows[0]
    d = Dev(wl)
    log(f"indexer fused {name}: T={q_idx.shape[0]}, k={k}")
    exp = _oracle_topk(wl, b, k=k, q_idx=q_idx, w=w, cu=np.array(cu))
    got = _gpu_topk(dsa, d, q_idx, w, cu, k, "fused")
    assert np.array_equal(got, exp), "fused top-k differs from the oracle"
    check_topk_rows_valid(got, wl.seq_lens, cu, k)
    ref = _gpu_topk(dsa, d, q_idx, w, cu, k, max(2, max(ql)))
    assert np.array_equal(got, ref), "fused and score-matrix paths differ"


def test_indexer_zero_rows(dsa):
    """T > 0 with no sequence rows at all (cu_q_lens = 0...): all -1."""
    wl = W.build(name="none", seed=6, S=2, kv_lens=[50, 60], PS=16, MP=4,
                 batches={"b": [0, 0, 0]}, H_idx=4, D_idx=32, k=8, with_mla=False)
    d = Dev(wl)
    q = W.f32_to_bf16(np.ones((5, 4, 32), np.float32))
    got = _gpu_topk(dsa, d, q, np.ones((5, 4), np.float32), [0, 0, 0], 8, 1)
    assert (got == -1).all()


# ----------------------------------------------------------------------------
# Union
# ----------------------------------------------------------------------------
def _gpu_union(dsa, topk, wl, cu, QB, u_max):
    torch = torch_mod()
    u, c, m = dsa.block_union(i32(topk, "cuda"), i32(wl.seq_lens, "cuda"), i32(cu, "cuda"),
                              wl.PS, wl.MP, QB, u_max)
    torch.cuda.synchronize()
    return u.cpu().numpy(), c.cpu().numpy(), m.cpu().numpy()


@pytest.mark.parametrize("QB", [16, 64])
def test_union_tiny(dsa, QB):
    wl = W.config(1, with_mla=False)
    b = wl.batches["extend"]
    tk = _oracle_topk(wl, b)
    log(f"union tiny QB={QB}")
    u, c, m = _gpu_union(dsa, tk, wl, b.cu_q_lens, QB, wl.u_max)
    eu, ec, em = oracle.block_union(tk, wl.seq_lens, b.cu_q_lens, wl.PS, wl.MP, QB, wl.u_max)
    assert np.array_equal(u, eu) and np.array_equal(c, ec) and np.array_equal(m, em)


UNION_CASES = {
    # name: (S, kv, PS, MP, q_lens, k, QB, u_max, fill)
    "ps16_qb3": (3, [100, 7, 64], 16, 8, [5, 2, 9], 12, 3, 64, 0.6),
    "ps48_qb8_lossless": (2, [400, 250], 48, 9, [20, 13], 40, 8, 18, 0.9),
    "ps64_qb64_lossy": (4, [900, 1200, 64, 333], 64, 20, [17, 30, 1, 40], 64, 64, 9, 0.8),
    "ps32_qb1": (2, [90, 150], 32, 5, [4, 6], 16, 1, 5, 1.0),
}


@pytest.mark.parametrize("name", sorted(UNION_CASES))
def test_union_cases(dsa, name):
    S, kv, PS, MP, ql, k, QB, u_max, fill = UNION_CASES[name]
    cu = np.concatenate([[0], np.cumsum(ql)])
    wl = W.build(name=name, seed=11, S=S, kv_lens=kv, PS=PS, MP=MP, batches={"b": cu}, H_idx=4,
                 D_idx=32, k=k, with_mla=False)
    tk = W.random_selection(wl.seq_lens, cu, k, 3, fill=fill, allow_out_of_range=True)
    tk = np.concatenate([tk, np.full((2, k), 5, np.int32)])  # rows past cu[S]: ignored
    log(f"union {name}")
    u, c, m = _gpu_union(dsa, tk, wl, cu, QB, u_max)
    eu, ec, em = oracle.block_union(tk, wl.seq_lens, cu, PS, MP, QB, u_max)
    assert np.array_equal(c, ec)
    assert np.array_equal(u, eu)
    assert np.array_equal(m, em)
    # sizes only (no membership pass): same units and counts, and a member
    # table handed in stays untouched
    torch = torch_mod()
    nqb = len(ec)
    out = (torch.full((nqb, u_max), -7, dtype=torch.int32, device="cuda"),
           torch.full((nqb,), -7, dtype=torch.int32, device="cuda"),
           torch.full((nqb, u_max, QB), 0x5A5A, dtype=torch.int64,
                      device="cuda").view(torch.uint64))
    u2, c2, m2 = dsa.block_union(i32(tk, "cuda"), i32(wl.seq_lens, "cuda"), i32(cu, "cuda"),
                                 PS, MP, QB, u_max, out=out, member=False)
    torch.cuda.synchronize()
    assert m2 is None
    assert np.array_equal(c2.cpu().numpy(), ec) and np.array_equal(u2.cpu().numpy(), eu)
    assert (out[2].cpu().numpy() == 0x5A5A).all()


# ----------------------------------------------------------------------------
# Sparse MLA
# ----------------------------------------------------------------------------
def _gpu_decode(dsa, d, q, kv, cu, topk, scale):
    torch = torch_mod()
    out = dsa.sparse_mla_decode(q, kv, d.page_table, d.seq_lens, i32(cu, "cuda"),
                                i32(topk, "cuda"), scale)
    torch.cuda.synchronize()
    return to_np(out)


def _gpu_extend(dsa, d, q, kv, cu, topk, scale, QB, u_max):
    torch = torch_mod()
    wl = d.wl
    cu_t = i32(cu, "cuda")
    u, c, m = dsa.block_union(i32(topk, "cuda"), d.seq_lens, cu_t, wl.PS, wl.MP, QB, u_max)
    out = dsa.sparse_mla_extend(q, kv, d.page_table, d.seq_lens, cu_t, u, c, m, QB, scale)
    torch.cuda.synchronize()
    return to_np(out), u.cpu().numpy(), c.cpu().numpy()


def _oracle_mla(wl, b, topk, layer=0, q=None, cu=None, kv=None):
    q = b.q_mla[layer] if q is None else q
    kv = wl.kv_cache[layer] if kv is None else kv
    return oracle.sparse_mla(bf16_to_f64(q), bf16_to_f64(kv), wl.page_table, wl.seq_lens,
                             b.cu_q_lens if cu is None else cu, topk, wl.sm_scale, wl.Dv)


@pytest.mark.parametrize("bname", ["decode", "extend"])
def test_mla_decode_tiny(dsa, bname):
    wl = W.config(1)
    b = wl.batches[bname]
    tk = _oracle_topk(wl, b)
    d = Dev(wl)
    log(f"mla decode tiny {bname}")
    got = _gpu_decode(dsa, d, bf16(b.q_mla[0], "cuda"), d.kv_cache[0], b.cu_q_lens, tk,
                      wl.sm_scale)
    check_attention(got, _oracle_mla(wl, b, tk), what=f"decode tiny {bname}")


MLA_CASES = {
    # name: (S, kv, PS, MP, q_lens, H, k, extra_rows, row_pad)
    "h16_ps64_multi": (3, [700, 64, 1500], 64, 24, [1, 3, 6], 16, 200, 2, 0),
    "h4_ps16": (2, [90, 333], 16, 24, [2, 5], 4, 40, 0, 64),
    "h32_ps32": (2, [500, 260], 32, 16, [4, 4], 32, 96, 1, 0),
    "h64_ps64": (1, [3000], 64, 50, [3], 64, 300, 0, 0),
    # a partial second 16-head block, PS = 48, padded rows, a row past the end
    "h20_ps48": (2, [777, 1300], 48, 30, [3, 2], 20, 260, 1, 8),
}


def _mla_case(name, seed=21):
    S, kv, PS, MP, ql, H, k, extra, pad = MLA_CASES[name]
    cu = np.concatenate([[0], np.cumsum(ql)])
    wl = W.build(name=name, seed=seed, S=S, kv_lens=kv, PS=PS, MP=MP, batches={"b": cu},
                 H_idx=4, D_idx=32, k=k, H_mla=H, extra_pages=1)
    b = wl.batches["b"]
    tk = W.random_selection(wl.seq_lens, cu, k, seed, fill=0.5, allow_out_of_range=True)
    q = b.q_mla[0]
    if extra:
        q = np.concatenate([q, q[:1].repeat(extra, 0)])
        tk = np.concatenate([tk, np.zeros((extra, k), np.int32)])
    tk[0, :] = -1  # an empty selection
    kvc = wl.kv_cache[0]
    if pad:
        kvc = kvc.with_columns(pad)
    return wl, b, cu, q, tk, kvc


@pytest.mark.parametrize("name", sorted(MLA_CASES))
def test_mla_decode_cases(dsa, name):
    wl, b, cu, q, tk, kvc = _mla_case(name)
    log(f"mla decode {name} T={q.shape[0]} row_stride={kvc.shape[-1]}")
    d = Dev(wl)
    got = _gpu_decode(dsa, d, bf16(q, "cuda"), kvc.to_torch("cuda"), cu, tk, wl.sm_scale)
    exp = oracle.sparse_mla(bf16_to_f64(q), bf16_to_f64(kvc), wl.page_table, wl.seq_lens, cu, tk,
                            wl.sm_scale, wl.Dv)
    assert (got[0] == 0).all()
    check_attention(got, exp, what=f"decode {name}")


@pytest.mark.parametrize("QB", [16, 64])
def test_mla_extend_tiny(dsa, QB):
    wl = W.config(1)
    b = wl.batches["extend"]
    tk = _oracle_topk(wl, b)
    d = Dev(wl)
    log(f"mla extend tiny QB={QB}")
    got, _, _ = _gpu_extend(dsa, d, bf16(b.q_mla[0], "cuda"), d.kv_cache[0], b.cu_q_lens, tk,
                            wl.sm_scale, QB, wl.u_max)
    check_attention(got, _oracle_mla(wl, b, tk), what=f"extend tiny QB={QB}")


EXTEND_CASES = {
    # name: (mla case, QB, u_max)  u_max=None -> lossless bound S*MP
    "h16_multi_qb4": ("h16_ps64_multi", 4, None),
    "h32_qb5_partial_tile": ("h32_ps32", 5, None),
    "h64_qb2": ("h64_ps64", 2, None),
    "h16_lossy_umax": ("h16_ps64_multi", 8, 5),
    "h4_ps16_qb16": ("h4_ps16", 16, None),
    "h20_ps48_qb3": ("h20_ps48", 3, None),
}


@pytest.mark.parametrize("name", sorted(EXTEND_CASES))
def test_mla_extend_cases(dsa, name):
    case, QB, u_max = EXTEND_CASES[name]
    wl, b, cu, q, tk, kvc = _mla_case(case, seed=31)
    if u_max is None:
        u_max = wl.S * wl.MP
    log(f"mla extend {name} QB={QB} u_max={u_max}")
    d = Dev(wl)
    got, units, counts = _gpu_extend(dsa, d, bf16(q, "cuda"), kvc.to_torch("cuda"), cu, tk,
                                     wl.sm_scale, QB, u_max)
    # the attended selection: entries whose page key survived the cap
    tk_eff = tk.copy()
    seq, _ = oracle.query_rows(wl.seq_lens, cu, tk.shape[0])
    for t in range(tk.shape[0]):
        bq = t // QB
        kept = set(units[bq, : min(int(counts[bq]), u_max)].tolist())
        for i, j in enumerate(tk[t]):
            if j >= 0 and (seq[t] < 0 or int(seq[t]) * wl.MP + int(j) // wl.PS not in kept):
                tk_eff[t, i] = -1
    if u_max < wl.S * wl.MP:
        assert (counts > u_max).any(), "lossy case did not overflow"
    exp = oracle.sparse_mla(bf16_to_f64(q), bf16_to_f64(kvc), wl.page_table, wl.seq_lens, cu,
                            tk_eff, wl.sm_scale, wl.Dv)
    check_attention(got, exp, what=f"extend {name}")


def test_extend_matches_decode(dsa):
    """The query-block kernel reproduces the per-row result for one selection."""
    wl, b, cu, q, tk, kvc = _mla_case("h16_ps64_multi", seed=41)
    d = Dev(wl)
    qd, kd = bf16(q, "cuda"), kvc.to_torch("cuda")
    dec = _gpu_decode(dsa, d, qd, kd, cu, tk, wl.sm_scale)
    ext, _, _ = _gpu_extend(dsa, d, qd, kd, cu, tk, wl.sm_scale, 4, wl.S * wl.MP)
    check_attention(ext, dec, what="extend vs decode")


def test_repeat_determinism(dsa):
    """Same inputs twice give identical bits (no races in LDS staging)."""
    wl = W.config(1)
    b = wl.batches["extend"]
    d = Dev(wl)
    tk1 = _gpu_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, wl.k, 32)
    tk2 = _gpu_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, wl.k, 32)
    assert np.array_equal(tk1, tk2)
    q = bf16(b.q_mla[0], "cuda")
    o1, _, _ = _gpu_extend(dsa, d, q, d.kv_cache[0], b.cu_q_lens, tk1, wl.sm_scale, 16, 32)
    o2, _, _ = _gpu_extend(dsa, d, q, d.kv_cache[0], b.cu_q_lens, tk1, wl.sm_scale, 16, 32)
    assert np.array_equal(o1, o2)


# ----------------------------------------------------------------------------
# Page-level selection: page top-k, page positions, attention over the pages
# ----------------------------------------------------------------------------
def _oracle_page_topk(wl, q_idx, w, cu, k_pages):
    return oracle.indexer_page_topk(bf16_to_f64(q_idx), w.astype(np.float64),
                                    bf16_to_f64(wl.idx_cache), wl.page_table, wl.seq_lens,
                                    np.asarray(cu), k_pages)


def _gpu_page_topk(dsa, d, q_idx, w, cu, k_pages, max_q_len):
    torch = torch_mod()
    out = dsa.indexer_page_topk(bf16(q_idx, "cuda"), f32(w, "cuda"), d.idx_cache, d.page_table,
                                d.seq_lens, i32(cu, "cuda"), k_pages, max_q_len)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("bname", ["decode", "extend"])
@pytest.mark.parametrize("path", ["rows", "tiles"])
def test_page_topk_tiny(dsa, bname, path):
    wl = W.config(1)
    b = wl.batches[bname]
    d = Dev(wl)
    mql = 1 if path == "rows" else max(2, _max_q_len(b.cu_q_lens))
    for kp in (1, 3, 16):
        log(f"page top-k tiny {bname} path={path} k_pages={kp}")
        got = _gpu_page_topk(dsa, d, b.q_idx, b.w, b.cu_q_lens, kp, mql)
        assert np.array_equal(got, _oracle_page_topk(wl, b.q_idx, b.w, b.cu_q_lens, kp))


PAGE_EDGE = {
    # name: (S, kv_lens, PS, MP, q_lens, H, D, k_pages, negative weights)
    "ps16_mixed_empty_seq": (3, [37, 200, 64], 16, 16, [1, 5, 0], 4, 32, 4, False),
    "ps32_negative_weights": (2, [77, 300], 32, 10, [3, 7], 8, 64, 3, True),
    "ps48_partial_pages": (2, [100, 1000], 48, 24, [2, 9], 32, 128, 5, True),
    "ps64_k_covers_all": (2, [1000, 4097], 64, 80, [4, 3], 32, 128, 100, False),
    "ps16_rows_above_8192_pages": (1, [132000], 16, 8256, [2], 4, 32, 64, True),
}


@pytest.mark.parametrize("name", sorted(PAGE_EDGE))
@pytest.mark.parametrize("path", ["rows", "tiles"])
def test_page_topk_edges(dsa, name, path):
    S, kv, PS, MP, ql, H, D, kp, neg = PAGE_EDGE[name]
    cu = np.concatenate([[0], np.cumsum(ql)]).tolist()
    wl = W.build(name=name, seed=91, S=S, kv_lens=kv, PS=PS, MP=MP, batches={"b": cu}, H_idx=H,
                 D_idx=D, k=kp, with_mla=False, extra_pages=1)
    b = wl.batches["b"]
    w = b.w.copy()
    if neg:  # negative head weights: page maxima below 0, masked slots must not count
        w[:, ::2] *= -1.0
    log(f"page top-k edge {name} path={path}")
    d = Dev(wl)
    mql = 1 if path == "rows" else max(2, max(ql))
    got = _gpu_page_topk(dsa, d, b.q_idx, w, cu, kp, mql)
    assert np.array_equal(got, _oracle_page_topk(wl, b.q_idx, w, cu, kp))


def test_page_tokens_and_attention_tiny(dsa):
    """Page top-k -> page positions -> attention (decode kernels, and the
    query-block path through the union) against the oracle's attention
    over the oracle's page positions."""
    torch = torch_mod()
    wl = W.config(1)
    d = Dev(wl)
    # k_pages 3, and 16: more than the 7 pages of the 100-token sequence, so
    # its rows carry -1 slots
    for kp, bname in ((3, "decode"), (3, "extend"), (16, "decode"), (16, "extend")):
        b = wl.batches[bname]
        bt = d.batch(bname)
        mql = max(1, _max_q_len(b.cu_q_lens))
        pages = dsa.indexer_page_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table,
                                      d.seq_lens, bt["cu"], kp, mql)
        tok = dsa.page_tokens(pages, wl.PS)
        torch.cuda.synchronize()
        exp_pages = _oracle_page_topk(wl, b.q_idx, b.w, b.cu_q_lens, kp)
        exp_tok = oracle.page_tokens(exp_pages, wl.PS)
        assert np.array_equal(pages.cpu().numpy(), exp_pages)
        assert np.array_equal(tok.cpu().numpy(), exp_tok)
        ref = oracle.sparse_mla(bf16_to_f64(b.q_mla[0]), bf16_to_f64(wl.kv_cache[0]),
                                wl.page_table, wl.seq_lens, b.cu_q_lens, exp_tok, wl.sm_scale,
                                wl.Dv)
        out = dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"],
                                    tok, wl.sm_scale)
        torch.cuda.synchronize()
        check_attention(to_np(out), ref, what=f"page attend {bname} (per query)")
        out = dsa.sparse_mla_decode_pages(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens,
                                          bt["cu"], pages, wl.sm_scale)
        torch.cuda.synchronize()
        check_attention(to_np(out), ref, what=f"page attend {bname} (page lists)")
        if bname == "extend" and kp == 3:
            for QB in wl.QB:
                u, c, m = dsa.block_union(tok, d.seq_lens, bt["cu"], wl.PS, wl.MP, QB, wl.u_max)
                out = dsa.sparse_mla_extend(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens,
                                            bt["cu"], u, c, m, QB, wl.sm_scale)
                torch.cuda.synchronize()
                check_attention(to_np(out), ref, what=f"page attend extend QB={QB}")


# ----------------------------------------------------------------------------
# Paged cache self-write
# ----------------------------------------------------------------------------
def _same_bits(a, b):
    return np.array_equal(np.nan_to_num(a, nan=-12345.0), np.nan_to_num(b, nan=-12345.0))


@pytest.mark.parametrize("bname", ["decode", "extend"])
def test_paged_write_tiny(dsa, bname):
    """New indexer keys (one call) and new latent rows (c_kv, then k_rope)
    written into the caches, compared slot by slot with the oracle; two
    extra rows past the last sequence are dropped. Then the attention over
    the updated latent cache matches the oracle's (write, then attend)."""
    torch = torch_mod()
    wl = W.config(1)
    b = wl.batches[bname]
    d = Dev(wl)
    bt = d.batch(bname)
    T = b.T + 2
    cu_t = bt["cu"]
    rng = np.random.default_rng(5)
    keys = rng.integers(-2, 3, size=(T, wl.D_idx)).astype(np.float32)
    lat = rng.standard_normal((T, 576)).astype(np.float32)
    keys_t = torch.from_numpy(keys).to("cuda").to(torch.bfloat16)
    lat_t = torch.from_numpy(lat).to("cuda").to(torch.bfloat16)
    idx0 = to_np(d.idx_cache)
    kv0 = to_np(d.kv_cache[0])
    dsa.paged_write(keys_t, d.idx_cache, d.page_table, d.seq_lens, cu_t)
    dsa.paged_write(lat_t[:, :512], d.kv_cache[0], d.page_table, d.seq_lens, cu_t, col0=0)
    dsa.paged_write(lat_t[:, 512:], d.kv_cache[0], d.page_table, d.seq_lens, cu_t, col0=512)
    torch.cuda.synchronize()
    exp_idx = oracle.paged_write(idx0, to_np(keys_t), 0, wl.page_table, wl.seq_lens, b.cu_q_lens)
    exp_kv = oracle.paged_write(kv0, to_np(lat_t), 0, wl.page_table, wl.seq_lens, b.cu_q_lens)
    assert _same_bits(to_np(d.idx_cache), exp_idx), "indexer cache after the write"
    assert _same_bits(to_np(d.kv_cache[0]), exp_kv), "latent cache after the write"
    # write, then attend: every causal position of each row, over the new cache
    seq, pos = oracle.query_rows(wl.seq_lens, b.cu_q_lens, b.T)
    sel = np.full((b.T, 256), -1, dtype=np.int32)
    for t in range(b.T):
        if seq[t] >= 0:
            n = oracle.n_valid_keys(wl.seq_lens[seq[t]], pos[t])
            sel[t, :min(n, 256)] = np.arange(min(n, 256))
    out = dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, cu_t,
                                i32(sel, "cuda"), wl.sm_scale)
    torch.cuda.synchronize()
    ref = oracle.sparse_mla(bf16_to_f64(b.q_mla[0]), exp_kv, wl.page_table, wl.seq_lens,
                            b.cu_q_lens, sel, wl.sm_scale, wl.Dv)
    check_attention(to_np(out), ref, what=f"write then attend ({bname})")
