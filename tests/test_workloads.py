"""The seeded input recipe: value sets, poison placement, selections."""
import numpy as np

import workloads as W


def test_bf16_roundtrip():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, np.nan, 0.0, -0.0], dtype=np.float32)
    b = W.f32_to_bf16(x)
    y = W.bf16_to_f32(b)
    assert np.isnan(y[4]) and y[0] == 1.0 and y[1] == -2.5 and y[2] == 3.140625
    # round to nearest even at the 8-bit mantissa boundary
    assert W.bf16_to_f32(W.f32_to_bf16(np.array([1.00390625], np.float32)))[0] == 1.0
    assert W.bf16_to_f32(W.f32_to_bf16(np.array([1.01171875], np.float32)))[0] == 1.015625


def test_tiny_recipe():
    wl = W.config(1)
    assert wl.S == 2 and wl.PS == 16 and wl.MP == 16 and wl.num_pages == 32
    assert sorted(wl.page_table.ravel().tolist()) == list(range(32))
    ic = W.bf16_to_f32(wl.idx_cache)
    kv = W.bf16_to_f32(wl.kv_cache[0])
    for s in range(2):
        for j in range(wl.MP * wl.PS):
            p, o = wl.page_table[s, j // wl.PS], j % wl.PS
            live = j < wl.seq_lens[s]
            assert np.isnan(ic[p, o]).all() != live
            assert np.isnan(kv[p, o]).all() != live
    vals = np.unique(ic[~np.isnan(ic)])
    assert set(vals.tolist()) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
    b = wl.batches["extend"]
    assert b.cu_q_lens.tolist() == [0, 0, 32] and b.T == 32
    assert set(np.unique(b.w).tolist()) <= {0.25, 0.5, 1.0, 2.0}
    assert not np.isnan(W.bf16_to_f32(b.q_mla[0])).any()


def test_seed_determinism():
    a = W.config(1)
    b = W.config(1)
    assert (a.idx_cache.rows == b.idx_cache.rows).all()
    assert (a.kv_cache[0].rows == b.kv_cache[0].rows).all()
    assert (a.idx_cache.dense() == b.idx_cache.dense()).all()
    assert (a.batches["extend"].q_idx == b.batches["extend"].q_idx).all()


def test_paged_cache_views():
    wl = W.config(1)
    dense = W.bf16_to_f64(wl.kv_cache[0].dense())
    view = wl.kv_cache[0].f64_view()
    pages = np.array([0, 3, 31, 7])
    offs = np.array([0, 15, 2, 9])
    got = view[pages, offs]
    exp = dense[pages, offs]
    assert np.array_equal(np.isnan(got), np.isnan(exp))
    assert np.array_equal(got[~np.isnan(got)], exp[~np.isnan(exp)])
    wide = wl.kv_cache[0].with_columns(64)
    assert wide.shape == (32, 16, 640) and np.isnan(W.bf16_to_f32(wide.dense()[..., 576:])).all()


def test_locality_selection():
    sl = np.array([3000])
    cu = np.array([0, 40])
    sel = W.locality_selection(sl, cu, 2048, 9)
    for t in range(40):
        p = 3000 - 40 + t
        row = sel[t]
        assert (row >= 0).all() and (np.diff(row) > 0).all() and row.max() <= p
        assert set(range(64)) <= set(row.tolist())
        assert set(range(p - 1023, p + 1)) <= set(row.tolist())
    short = W.locality_selection(np.array([100]), np.array([0, 2]), 2048, 1)
    assert short[0, :99].tolist() == list(range(99)) and (short[0, 99:] == -1).all()
