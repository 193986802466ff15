"""Pins for the CPU oracle (no GPU).

Each pin checks the oracle against something other than itself: pure-Python
brute force on tiny inputs (rank counting instead of sorting, set scans
instead of the oracle's dictionary), hand-worked fixtures in
``tests/golden/``, closed forms, a textbook dense attention (SciPy softmax),
and invariants. ``test_planted_mistakes`` then plants plausible mistakes in
the oracle's building blocks and requires at least one pin to fail for each.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import oracle.dsa as odsa
import workloads as W
from workloads import bf16_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(x):
    return np.array([[[float(v) for v in r] for r in p] for p in x], dtype=np.float64)


# ----------------------------------------------------------------------------
# Small seeded workloads
# ----------------------------------------------------------------------------
def micro(seed, *, S=2, PS=4, MP=5, H=3, D=4, k=6, q_lens=(3, 2), H_mla=2, Dk=8, Dv=5):
    rng = np.random.default_rng(seed)
    kv = [int(rng.integers(ql, MP * PS + 1)) for ql in q_lens]
    cu = [0]
    for ql in q_lens:
        cu.append(cu[-1] + ql)
    return W.build(name=f"micro{seed}", seed=seed, S=S, kv_lens=kv, PS=PS, MP=MP,
                   batches={"b": cu}, H_idx=H, D_idx=D, k=k, H_mla=H_mla, Dk=Dk, Dv=Dv,
                   sm_scale=0.4, extra_pages=1)


def py_abs_positions(seq_lens, cu, T):
    """Independent restatement of the row bookkeeping, in plain Python."""
    res = []
    for t in range(T):
        found = None
        for s in range(len(seq_lens)):
            if cu[s] <= t < cu[s + 1]:
                found = (s, int(seq_lens[s]) - (cu[s + 1] - cu[s]) + (t - cu[s]))
        res.append(found)
    return res


def py_key(cache, pt, s, j):
    PS = len(cache[0])
    return cache[pt[s][j // PS]][j % PS]


def brute_topk(q, w, cache, pt, seq_lens, cu, k):
    """Pure-Python top-k by rank counting (no sort)."""
    T = len(q)
    out = [[-1] * k for _ in range(T)]
    for t, info in enumerate(py_abs_positions(seq_lens, cu, T)):
        if info is None:
            continue
        s, a = info
        n = max(0, min(int(seq_lens[s]), a + 1))
        sc = []
        for j in range(n):
            kj = py_key(cache, pt, s, j)
            tot = 0.0
            for h in range(len(q[t])):
                d = sum(q[t][h][x] * kj[x] for x in range(len(kj)))
                tot += w[t][h] * (d if d > 0 else 0.0)
            sc.append(tot)
        for j in range(n):
            rank = sum(1 for i in range(n) if sc[i] > sc[j] or (sc[i] == sc[j] and i < j))
            if rank < k:
                out[t][rank] = j
    return out


def _indexer_inputs(wl, bname):
    b = wl.batches[bname]
    return (bf16_to_f64(b.q_idx), b.w.astype(np.float64), bf16_to_f64(wl.idx_cache),
            wl.page_table, wl.seq_lens, b.cu_q_lens)


# ----------------------------------------------------------------------------
# Indexer pins
# ----------------------------------------------------------------------------
def pin_indexer_golden():
    g = _load("indexer_hand.json")
    cache = _arr(g["idx_cache"])
    pt = np.array(g["page_table"])
    for k, exp in g["expected"].items():
        got = oracle.indexer_topk(np.array(g["q"], float), np.array(g["w"], float), cache, pt,
                                  np.array(g["seq_lens"]), np.array(g["cu_q_lens"]), int(k))
        assert got.tolist() == exp, (k, got.tolist(), exp)


def pin_indexer_bruteforce():
    for seed in range(6):
        wl = micro(seed)
        q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
        got = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
        exp = brute_topk(q.tolist(), w.tolist(), cache.tolist(), pt.tolist(), sl.tolist(),
                         cu.tolist(), wl.k)
        assert got.tolist() == exp, seed


def pin_indexer_tiny_bruteforce():
    wl = W.config(1, with_mla=False)
    for bname in ("decode", "extend"):
        q, w, cache, pt, sl, cu = _indexer_inputs(wl, bname)
        rows = [0, 1] if bname == "decode" else [0, 17, 31]
        got = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k, rows=rows)
        exp = brute_topk(q.tolist(), w.tolist(), cache.tolist(), pt.tolist(), sl.tolist(),
                         cu.tolist(), wl.k)
        for t in rows:
            assert got[t].tolist() == exp[t], (bname, t)


def pin_indexer_zero_query():
    """q = 0 makes every score 0: the result is the tie order 0, 1, 2, ..."""
    wl = micro(11, k=9)
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
    got = oracle.indexer_topk(np.zeros_like(q), w, cache, pt, sl, cu, wl.k)
    for t, (s, a) in enumerate(py_abs_positions(sl, cu, q.shape[0])):
        n = min(int(sl[s]), a + 1)
        m = min(wl.k, n)
        assert got[t].tolist() == list(range(m)) + [-1] * (wl.k - m)


def pin_indexer_single_head():
    """H = 1, w = 1: ranking by relu(q . k), checked with Python's sorted()."""
    wl = micro(12, H=1, k=7)
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
    w = np.ones_like(w)
    got = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
    for t, (s, a) in enumerate(py_abs_positions(sl, cu, q.shape[0])):
        n = min(int(sl[s]), a + 1)
        vals = [max(0.0, float(np.dot(q[t, 0], py_key(cache, pt, s, j)))) for j in range(n)]
        order = sorted(range(n), key=lambda j: (-vals[j], j))[: wl.k]
        assert got[t].tolist() == order + [-1] * (wl.k - len(order))


def pin_indexer_k_covers_all():
    """k >= n_valid: every causal position appears exactly once, then -1."""
    wl = micro(13, k=40)
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
    got = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
    for t, (s, a) in enumerate(py_abs_positions(sl, cu, q.shape[0])):
        n = min(int(sl[s]), a + 1)
        row = got[t].tolist()
        assert sorted(row[:n]) == list(range(n)) and row[n:] == [-1] * (wl.k - n)


def check_topk_invariants(topk, q, w, cache, pt, sl, cu, k, rows):
    for t in rows:
        info = py_abs_positions(sl, cu, q.shape[0])[t]
        row = topk[t]
        if info is None:
            assert (row == -1).all()
            continue
        s, a = info
        n = max(0, min(int(sl[s]), a + 1))
        m = min(k, n)
        assert (row[:m] >= 0).all() and (row[m:] == -1).all()  # -1 count = k - min(k, n)
        assert (row[:m] <= a).all() and (row[:m] < sl[s]).all()  # causality
        assert len(set(row[:m].tolist())) == m
        # scores along the row are non-increasing; equal scores by ascending position
        ks = np.array([py_key(cache, pt, s, int(j)) for j in row[:m]], dtype=np.float64)
        sc = np.maximum(ks @ q[t].T, 0) @ w[t]
        assert (np.diff(sc) <= 0).all()
        ties = np.diff(sc) == 0
        assert (np.diff(row[:m])[ties] > 0).all()
        # nothing left out scores above the last kept one
        if m < n:
            rest = sorted(set(range(n)) - set(row[:m].tolist()))
            kr = np.array([py_key(cache, pt, s, j) for j in rest], dtype=np.float64)
            sr = np.maximum(kr @ q[t].T, 0) @ w[t]
            last = sc[-1]
            assert (sr <= last).all()
            assert all(j > row[m - 1] for j, v in zip(rest, sr) if v == last)


def pin_indexer_invariants_tiny():
    wl = W.config(1, with_mla=False)
    for bname in ("decode", "extend"):
        q, w, cache, pt, sl, cu = _indexer_inputs(wl, bname)
        got = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
        check_topk_invariants(got, q, w, cache, pt, sl, cu, wl.k, range(q.shape[0]))


def pin_indexer_page_permutation():
    """Permuting physical pages together with the page table changes nothing."""
    wl = W.config(1, with_mla=False)
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "extend")
    base = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
    perm = np.random.default_rng(5).permutation(cache.shape[0])  # new page p holds old perm[p]
    inv = np.argsort(perm)
    got = oracle.indexer_topk(q, w, cache[perm], inv[pt], sl, cu, wl.k)
    assert (got == base).all()


def pin_indexer_weight_scaling():
    """Scaling every w by 2**m scales every score exactly: same selection."""
    wl = W.config(1, with_mla=False)
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "extend")
    base = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
    for m in (-3, 4):
        assert (oracle.indexer_topk(q, w * 2.0 ** m, cache, pt, sl, cu, wl.k) == base).all()


def pin_indexer_outside_rows():
    """Rows beyond the last sequence's queries are all -1; an empty sequence
    (q_len 0) contributes no rows."""
    wl = micro(14, q_lens=(0, 3))
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
    q2 = np.concatenate([q, q[:2]])  # two rows past cu[-1]
    w2 = np.concatenate([w, w[:2]])
    got = oracle.indexer_topk(q2, w2, cache, pt, sl, cu, wl.k)
    assert (got[-2:] == -1).all()
    exp = brute_topk(q.tolist(), w.tolist(), cache.tolist(), pt.tolist(), sl.tolist(),
                     cu.tolist(), wl.k)
    assert got[:-2].tolist() == exp


# ----------------------------------------------------------------------------
# Union pins
# ----------------------------------------------------------------------------
def brute_union(topk, sl, cu, PS, MP, QB, u_max):
    """Scan every possible key in increasing order (no set/dict)."""
    T = len(topk)
    info = py_abs_positions(sl, cu, T)
    nqb = (T + QB - 1) // QB
    units, counts, member = [], [], []
    for b in range(nqb):
        rows = [t for t in range(b * QB, min(T, (b + 1) * QB)) if info[t] is not None]
        present = []
        for key in range(len(sl) * MP):
            s, page = divmod(key, MP)
            hit = any(info[t][0] == s and any(0 <= j < MP * PS and j // PS == page for j in topk[t])
                      for t in rows)
            if hit:
                present.append(key)
        counts.append(len(present))
        kept = present[:u_max]
        units.append(kept + [-1] * (u_max - len(kept)))
        mb = [[0] * QB for _ in range(u_max)]
        for i, key in enumerate(kept):
            s, page = divmod(key, MP)
            for t in rows:
                if info[t][0] != s:
                    continue
                for j in topk[t]:
                    if 0 <= j < MP * PS and j // PS == page:
                        mb[i][t - b * QB] |= 1 << (j - page * PS)
        member.append(mb)
    return units, counts, member


def _union_case(seed, QB, u_max, fill=0.6):
    wl = micro(seed, S=3, PS=4, MP=5, q_lens=(3, 0, 4), k=5)
    b = wl.batches["b"]
    sel = W.random_selection(wl.seq_lens, b.cu_q_lens, wl.k, seed, fill=fill)
    return wl, b, sel


def pin_union_bruteforce():
    for seed, QB, u_max in [(1, 2, 16), (2, 3, 7), (3, 4, 3), (4, 16, 48), (5, 1, 2)]:
        wl, b, sel = _union_case(seed, QB, u_max)
        u, c, m = oracle.block_union(sel, wl.seq_lens, b.cu_q_lens, wl.PS, wl.MP, QB, u_max)
        eu, ec, em = brute_union(sel.tolist(), wl.seq_lens, b.cu_q_lens.tolist(), wl.PS, wl.MP,
                                 QB, u_max)
        assert u.tolist() == eu and c.tolist() == ec
        assert m.astype(np.int64).tolist() == em


def pin_union_invariants():
    wl = W.config(1, with_mla=False)
    q, w, cache, pt, sl, cu = _indexer_inputs(wl, "extend")
    tk = oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)
    for QB in wl.QB:
        u, c, m = oracle.block_union(tk, sl, cu, wl.PS, wl.MP, QB, wl.u_max)
        for b in range(u.shape[0]):
            n = min(int(c[b]), wl.u_max)
            assert (np.diff(u[b, :n]) > 0).all() and (u[b, n:] == -1).all()
            assert (m[b, n:] == 0).all()
            for qi in range(QB):
                t = b * QB + qi
                nsel = int((tk[t] >= 0).sum()) if t < tk.shape[0] else 0
                pop = sum(bin(int(x)).count("1") for x in m[b, :, qi])
                assert pop == nsel


# ----------------------------------------------------------------------------
# Sparse-MLA pins
# ----------------------------------------------------------------------------
def _mla_inputs(wl, bname, layer=0):
    b = wl.batches[bname]
    return (bf16_to_f64(b.q_mla[layer]), bf16_to_f64(wl.kv_cache[layer]), wl.page_table,
            wl.seq_lens, b.cu_q_lens)


def pin_mla_golden():
    g = _load("mla_hand.json")
    out = oracle.sparse_mla(np.array(g["q"], float), _arr(g["kv_cache"]), np.array(g["page_table"]),
                            np.array(g["seq_lens"]), np.array(g["cu_q_lens"]),
                            np.array(g["topk"]), g["sm_scale"], g["v_dim"])
    assert np.allclose(out, np.array(g["expected"]), rtol=0, atol=1e-12), out


def pin_mla_sparse_equals_dense():
    """Selecting every causal position equals dense causal attention
    (textbook softmax(q K^T * scale) V with SciPy's softmax)."""
    wl = W.config(1)
    k_all = 256
    for bname in ("decode", "extend"):
        q, kv, pt, sl, cu = _mla_inputs(wl, bname)
        qi, wi, ci, _, _, _ = _indexer_inputs(wl, bname)
        tk = oracle.indexer_topk(qi, wi, ci, pt, sl, cu, k_all)
        out = oracle.sparse_mla(q, kv, pt, sl, cu, tk, wl.sm_scale, wl.Dv)
        for t, (s, a) in enumerate(py_abs_positions(sl, cu, q.shape[0])):
            rows = np.array([py_key(kv, pt, s, j) for j in range(a + 1)])
            logits = np.einsum("hd,nd->hn", q[t], rows) * wl.sm_scale
            p = scipy.special.softmax(logits, axis=-1)
            ref = np.einsum("hn,nd->hd", p, rows[:, : wl.Dv])
            assert np.allclose(out[t], ref, rtol=1e-10, atol=1e-12)


def pin_mla_closed_forms():
    wl = micro(21, H_mla=3, Dk=8, Dv=5)
    q, kv, pt, sl, cu = _mla_inputs(wl, "b")
    T = q.shape[0]
    info = py_abs_positions(sl, cu, T)
    # single valid selection -> that row's value part
    tk = np.full((T, 4), -1, dtype=np.int32)
    for t, (s, a) in enumerate(info):
        tk[t, 2] = a  # the query's own position
    out = oracle.sparse_mla(q, kv, pt, sl, cu, tk, 0.4, 5)
    for t, (s, a) in enumerate(info):
        assert np.allclose(out[t], np.broadcast_to(py_key(kv, pt, s, a)[:5], (3, 5)), atol=1e-12)
    # all selected value parts equal c -> output c, whatever the logits
    c = np.arange(5, dtype=np.float64) - 2.0
    kv2 = kv.copy()
    kv2[..., :5] = c
    tk = W.random_selection(sl, cu, 4, 3, fill=1.0)
    out = oracle.sparse_mla(q, kv2, pt, sl, cu, tk, 0.4, 5)
    for t in range(T):
        assert np.allclose(out[t], c, atol=1e-12)
    # huge scale -> the arg-max row's value part
    tk = W.random_selection(sl, cu, 4, 4, fill=1.0)
    out = oracle.sparse_mla(q, kv, pt, sl, cu, tk, 1e6, 5)
    for t, (s, a) in enumerate(info):
        js = [int(j) for j in tk[t] if j >= 0]
        for h in range(3):
            best = max(js, key=lambda j: float(np.dot(q[t, h], py_key(kv, pt, s, j))))
            assert np.allclose(out[t, h], py_key(kv, pt, s, best)[:5], atol=1e-9)
    # empty selection -> zeros
    out = oracle.sparse_mla(q, kv, pt, sl, cu, np.full((T, 4), -1, np.int32), 0.4, 5)
    assert (out == 0).all()


def brute_mla(q, kv, pt, sl, cu, tk, scale, v_dim):
    T = len(q)
    out = [[[0.0] * v_dim for _ in range(len(q[0]))] for _ in range(T)]
    for t, info in enumerate(py_abs_positions(sl, cu, T)):
        if info is None:
            continue
        s, a = info
        js = [j for j in tk[t] if 0 <= j < sl[s] and j <= a]
        if not js:
            continue
        for h in range(len(q[t])):
            rows = [py_key(kv, pt, s, j) for j in js]
            lg = [scale * sum(q[t][h][d] * r[d] for d in range(len(q[t][h]))) for r in rows]
            mx = max(lg)
            e = [math.exp(x - mx) for x in lg]
            z = sum(e)
            for d in range(v_dim):
                out[t][h][d] = sum(e[i] * rows[i][d] for i in range(len(rows))) / z
    return out


def pin_mla_bruteforce():
    for seed in range(4):
        wl = micro(30 + seed, H_mla=2, Dk=8, Dv=5)
        q, kv, pt, sl, cu = _mla_inputs(wl, "b")
        tk = W.random_selection(sl, cu, 6, seed, fill=0.8, allow_out_of_range=True)
        out = oracle.sparse_mla(q, kv, pt, sl, cu, tk, 0.4, 5)
        exp = brute_mla(q.tolist(), kv.tolist(), pt.tolist(), sl.tolist(), cu.tolist(),
                        tk.tolist(), 0.4, 5)
        assert np.allclose(out, np.array(exp), rtol=1e-12, atol=1e-12), seed


def pin_mla_softmax_rows_sum_to_one():
    wl = W.config(1)
    q, kv, pt, sl, cu = _mla_inputs(wl, "extend")
    tk = W.locality_selection(sl, cu, 32, 7, sinks=4, window=8)
    _, pos = oracle.query_rows(sl, cu, q.shape[0])
    for t in range(q.shape[0]):
        sel = oracle.valid_selection(tk[t], sl[1], pos[t])
        rows = oracle.gather_rows(kv, pt, 1, sel)
        p = oracle.softmax(wl.sm_scale * q[t] @ rows.T)
        assert np.allclose(p.sum(-1), 1.0, atol=1e-12) and (p >= 0).all()


def py_scores(q, w, cache, pt, s, t, n):
    """Pure-Python scores of row t against positions 0 .. n-1 of sequence s."""
    sc = []
    for j in range(n):
        kj = py_key(cache, pt, s, j)
        tot = 0.0
        for h in range(len(q[t])):
            d = sum(q[t][h][x] * kj[x] for x in range(len(kj)))
            tot += w[t][h] * (d if d > 0 else 0.0)
        sc.append(tot)
    return sc


def brute_page_topk(q, w, cache, pt, seq_lens, cu, k_pages):
    """Pure-Python page top-k: explicit page maxima, rank counting."""
    PS = len(cache[0])
    T = len(q)
    out = [[-1] * k_pages for _ in range(T)]
    for t, info in enumerate(py_abs_positions(seq_lens, cu, T)):
        if info is None:
            continue
        s, a = info
        n = max(0, min(int(seq_lens[s]), a + 1))
        sc = py_scores(q, w, cache, pt, s, t, n)
        npg = (n + PS - 1) // PS
        ps = [max(sc[p * PS: min((p + 1) * PS, n)]) for p in range(npg)]
        for p in range(npg):
            rank = sum(1 for i in range(npg) if ps[i] > ps[p] or (ps[i] == ps[p] and i < p))
            if rank < k_pages:
                out[t][rank] = p
    return out


def pin_page_topk_bruteforce():
    """Micro workloads with partial last pages, positive head weights and
    mixed-sign ones (negative scores: a masked position must never count
    as 0 in a page's maximum)."""
    for seed in range(6):
        wl = micro(seed)
        q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
        for sign in (np.ones(w.shape[1]), np.array([-1.0, 1.0, -1.0])):
            ws = w * sign[None, :]
            for kp in (1, 2, 7):
                got = oracle.indexer_page_topk(q, ws, cache, pt, sl, cu, kp)
                exp = brute_page_topk(q.tolist(), ws.tolist(), cache.tolist(), pt.tolist(),
                                      sl.tolist(), cu.tolist(), kp)
                assert got.tolist() == exp, (seed, kp)


def pin_page_topk_unit_pages_is_token_topk():
    """With one position per page the page top-k is the token top-k."""
    for seed in range(3):
        wl = micro(100 + seed, PS=1, MP=20)
        q, w, cache, pt, sl, cu = _indexer_inputs(wl, "b")
        got = oracle.indexer_page_topk(q, w, cache, pt, sl, cu, wl.k)
        assert np.array_equal(got, oracle.indexer_topk(q, w, cache, pt, sl, cu, wl.k)), seed


def pin_page_topk_invariants_tiny():
    """Tiny workload (PS 16): padding count, valid pages only, page scores
    non-increasing, and the best token's page first."""
    wl = W.config(1, with_mla=False)
    for bname in ("decode", "extend"):
        q, w, cache, pt, sl, cu = _indexer_inputs(wl, bname)
        T = q.shape[0]
        kp = 3
        got = oracle.indexer_page_topk(q, w, cache, pt, sl, cu, kp)
        seq, pos = oracle.query_rows(sl, cu, T)
        for t in range(T):
            if seq[t] < 0:
                assert (got[t] == -1).all()
                continue
            n = oracle.n_valid_keys(sl[seq[t]], pos[t])
            npg = -(-n // wl.PS)
            row = got[t]
            assert (row[min(kp, npg):] == -1).all() and (row[:min(kp, npg)] >= 0).all()
            assert (row[:min(kp, npg)] < npg).all() and len(set(row[:min(kp, npg)])) == min(kp, npg)
            sc = oracle.indexer_score_row(q, w, cache, pt, sl, cu, t)
            pmax = [sc[p * wl.PS:(p + 1) * wl.PS].max() for p in row[:min(kp, npg)]]
            assert all(pmax[i] >= pmax[i + 1] for i in range(len(pmax) - 1))
            assert row[0] == int(np.argmax(sc)) // wl.PS or pmax[0] == sc.max()


def pin_page_tokens():
    pages = np.array([[2, 0, -1], [-1, -1, -1]])
    exp = [[8, 9, 10, 11, 0, 1, 2, 3, -1, -1, -1, -1], [-1] * 12]
    assert oracle.page_tokens(pages, 4).tolist() == exp


def pin_paged_write_bruteforce():
    """Plain-Python slot arithmetic on micro workloads (with rows past the
    last sequence); everything not written stays as it was, and reading the
    written positions back through the page table gives the new rows."""
    for seed in range(4):
        wl = micro(200 + seed, q_lens=(3, 0, 2), S=3)
        b = wl.batches["b"]
        cache = bf16_to_f64(wl.idx_cache)
        T = int(b.cu_q_lens[-1]) + 2  # two rows in no sequence
        rows = np.arange(T * 2, dtype=np.float64).reshape(T, 2) + 1000.0
        got = oracle.paged_write(cache, rows, 1, wl.page_table, wl.seq_lens, b.cu_q_lens)
        exp = cache.copy()
        cu = [int(x) for x in b.cu_q_lens]
        PS = cache.shape[1]
        for s in range(wl.S):
            q0, q1 = cu[s], cu[s + 1]
            for t in range(q0, q1):
                a = int(wl.seq_lens[s]) - (q1 - q0) + (t - q0)
                if 0 <= a < int(wl.seq_lens[s]):
                    pg = int(wl.page_table[s][a // PS])
                    exp[pg, a % PS, 1] = rows[t, 0]
                    exp[pg, a % PS, 2] = rows[t, 1]
        assert np.array_equal(np.nan_to_num(got, nan=-7.0), np.nan_to_num(exp, nan=-7.0)), seed
        seq, pos = oracle.query_rows(wl.seq_lens, b.cu_q_lens, T)
        for t in range(T):
            if seq[t] >= 0:
                back = oracle.gather_rows(got, wl.page_table, int(seq[t]), [int(pos[t])])[0]
                assert np.array_equal(back[1:3], rows[t])
    # page-table entries that name no page of the cache (-1, or past the
    # pool) give those positions no slot: nothing at all is written for them
    wl = micro(210, q_lens=(3, 0, 2), S=3)
    b = wl.batches["b"]
    cache = bf16_to_f64(wl.idx_cache)
    P, PS = cache.shape[0], cache.shape[1]
    T = int(b.cu_q_lens[-1])
    rows = np.arange(T * 2, dtype=np.float64).reshape(T, 2) + 500.0
    seq, pos = oracle.query_rows(wl.seq_lens, b.cu_q_lens, T)
    pt = np.array(wl.page_table, copy=True)
    t_bad, t_far = int(b.cu_q_lens[0]), int(b.cu_q_lens[2])  # first rows of sequences 0 and 2
    pt[int(seq[t_bad]), int(pos[t_bad]) // PS] = -1
    pt[int(seq[t_far]), int(pos[t_far]) // PS] = P + 3
    got = oracle.paged_write(cache, rows, 1, pt, wl.seq_lens, b.cu_q_lens)
    exp = cache.copy()
    for t in range(T):
        s, a = int(seq[t]), int(pos[t])
        if s < 0 or not (0 <= a < int(wl.seq_lens[s])):
            continue
        pg = int(pt[s][a // PS])
        if 0 <= pg < P:
            exp[pg, a % PS, 1:3] = rows[t]
    assert np.array_equal(np.nan_to_num(got, nan=-7.0), np.nan_to_num(exp, nan=-7.0))
    # the -1 entry must not reach the last page (a negative index would)
    assert np.array_equal(np.nan_to_num(got[P - 1], nan=-7.0), np.nan_to_num(exp[P - 1], nan=-7.0))


PINS = [
    pin_paged_write_bruteforce,
    pin_page_topk_bruteforce, pin_page_topk_unit_pages_is_token_topk,
    pin_page_topk_invariants_tiny, pin_page_tokens,
    pin_indexer_golden, pin_indexer_bruteforce, pin_indexer_tiny_bruteforce,
    pin_indexer_zero_query, pin_indexer_single_head, pin_indexer_k_covers_all,
    pin_indexer_invariants_tiny, pin_indexer_page_permutation, pin_indexer_weight_scaling,
    pin_indexer_outside_rows, pin_union_bruteforce, pin_union_invariants, pin_mla_golden,
    pin_mla_sparse_equals_dense, pin_mla_closed_forms, pin_mla_bruteforce,
    pin_mla_softmax_rows_sum_to_one,
]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# Planted mistakes: every one must be caught by at least one pin
# ----------------------------------------------------------------------------
def _m_no_relu(dots, w):
    return dots @ w


def _m_no_weights(dots, w):
    return np.maximum(dots, 0.0).sum(axis=1)


def _m_tie_high(scores):
    return np.lexsort((-np.arange(scores.shape[0]), -scores))


def _m_ascending(scores):
    return np.lexsort((np.arange(scores.shape[0]), scores))


def _m_causal_strict(kv_len, abs_q):
    return int(max(0, min(int(kv_len), int(abs_q))))


def _m_no_causal(kv_len, abs_q):
    return int(max(0, int(kv_len)))


def _m_gather_offset(cache, page_table, s, positions):
    PS = cache.shape[1]
    positions = np.asarray(positions, dtype=np.int64)
    return cache[page_table[s, positions // PS], (positions + 1) % PS]


def _m_gather_no_table(cache, page_table, s, positions):
    PS = cache.shape[1]
    positions = np.asarray(positions, dtype=np.int64)
    MP = page_table.shape[1]
    return cache[(s * MP + positions // PS) % cache.shape[0], positions % PS]


def _m_key_ps(s, j, MP, PS):
    return int(s) * PS + int(j) // PS


def _m_bit_page(j, PS):
    return 1 << (int(j) // PS % 64)


def _m_sel_no_causal(sel, kv_len, abs_q):
    sel = np.asarray(sel, dtype=np.int64)
    return sel[(sel >= 0) & (sel < kv_len)]


def _m_attend_no_scale(q_t, rows, sm_scale, v_dim):
    return odsa.softmax(q_t @ rows.T) @ rows[:, :v_dim]


def _m_attend_rope_value(q_t, rows, sm_scale, v_dim):
    return odsa.softmax(sm_scale * (q_t @ rows.T)) @ rows[:, -v_dim:]


def _m_attend_nope_only(q_t, rows, sm_scale, v_dim):
    return odsa.softmax(sm_scale * (q_t[:, :v_dim] @ rows[:, :v_dim].T)) @ rows[:, :v_dim]


def _m_softmax_wrong_axis(logits):
    m = logits.max(axis=0, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=0, keepdims=True)


def _m_page_pool_mean(scores, PS):
    n = scores.shape[0]
    npg = -(-n // PS)
    return np.array([scores[p * PS:(p + 1) * PS].mean() for p in range(npg)])


def _m_page_pool_masked_zero(scores, PS):
    n = scores.shape[0]
    npg = -(-n // PS)
    padded = np.zeros(npg * PS)
    padded[:n] = scores
    return padded.reshape(npg, PS).max(axis=1)


def _m_query_rows_shift(seq_lens, cu_q_lens, T):
    seq, pos = _ORIG["query_rows"](seq_lens, cu_q_lens, T)
    return seq, np.where(pos >= 0, pos - 1, pos)


_ORIG = {"query_rows": odsa.query_rows}

MUTANTS = {
    "no_relu": ("head_mix", _m_no_relu),
    "no_weights": ("head_mix", _m_no_weights),
    "tie_to_higher_position": ("canonical_order", _m_tie_high),
    "ascending_order": ("canonical_order", _m_ascending),
    "causal_strict": ("n_valid_keys", _m_causal_strict),
    "no_causal_bound": ("n_valid_keys", _m_no_causal),
    "gather_wrong_offset": ("gather_rows", _m_gather_offset),
    "gather_ignores_table": ("gather_rows", _m_gather_no_table),
    "union_key_stride": ("unit_key", _m_key_ps),
    "member_bit_page": ("member_bit", _m_bit_page),
    "attend_no_causal": ("valid_selection", _m_sel_no_causal),
    # (dropping only the j < kv_len term is not a mistake: with derived
    # positions abs_q <= kv_len - 1, so the causal term already implies it)
    "attend_no_scale": ("attend", _m_attend_no_scale),
    "attend_value_slice": ("attend", _m_attend_rope_value),
    "attend_drops_rope": ("attend", _m_attend_nope_only),
    "softmax_axis": ("softmax", _m_softmax_wrong_axis),
    "abs_position_shift": ("query_rows", _m_query_rows_shift),
    "page_pool_mean": ("page_pool", _m_page_pool_mean),
    "page_pool_masked_as_zero": ("page_pool", _m_page_pool_masked_zero),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(odsa, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # noqa: BLE001 - a crash also counts as caught
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
