"""GPU parity of the paged cache self-write and of the layer runner at the
chunked-extend size (4 requests x (12288 + 1024), T = 4096).

* dsa_paged_write_layer writes the chunk's indexer keys and latent rows into
  caches whose chunk slots were poisoned, with two page-table entries that
  name no page of the cache (-1 and one past the pool): every slot of both
  caches, written or not, is compared with the oracle's cache bit for bit.
* extend_layers runs four layers (full, shared, full, shared) with the
  self-write first, the indexer and the unions on full layers only, and the
  attention chosen by dsa_extend_attend_plan (or forced: per query, QB 64,
  QB 256); top-k is compared with the oracle on sampled rows of each full
  layer and the attention of every layer on sampled rows.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_helpers import (Dev, bf16, check_attention, check_topk_rows_valid, i32, log, to_np,
                         torch_mod)
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


def _chunk_rows(cache, wl, cu):
    """bf16 bits [T, D] of the workload cache at each packed row's own
    position (the rows the self-write puts back)."""
    T = int(cu[-1])
    dense = cache.dense().reshape(-1, cache.D)
    seq, pos = oracle.query_rows(wl.seq_lens, cu, T)
    slots = np.array([int(wl.page_table[s, p // wl.PS]) * wl.PS + p % wl.PS
                      for s, p in zip(seq, pos)], dtype=np.int64)
    return dense[slots], slots


def _poisoned(t, slots):
    """Device cache with the given flat slots overwritten by NaN."""
    torch = torch_mod()
    P, PS, D = t.shape
    flat = t.view(P * PS, D)
    flat[torch.from_numpy(slots).to(t.device)] = float("nan")
    return t


def test_paged_write_layer_config4_every_slot(dsa):
    torch = torch_mod()
    wl = W.config(4)
    b = wl.batches["extend"]
    cu = b.cu_q_lens
    T = b.T
    new_idx, slots = _chunk_rows(wl.idx_cache, wl, cu)
    new_kv, _ = _chunk_rows(wl.kv_cache[0], wl, cu)
    pt = np.array(wl.page_table, copy=True)
    P = wl.num_pages
    seq, pos = oracle.query_rows(wl.seq_lens, cu, T)
    t1, t2 = int(cu[1]) + 100, int(cu[2]) + 700  # rows of sequences 1 and 2
    pt[int(seq[t1]), int(pos[t1]) // wl.PS] = -1
    pt[int(seq[t2]), int(pos[t2]) // wl.PS] = P + 5
    log(f"paged write layer: T={T}, page entries -1 and {P + 5} at rows {t1}, {t2}")
    d = Dev(wl, layers=1)
    icache = _poisoned(d.idx_cache, slots)
    kcache = _poisoned(d.kv_cache[0], slots)
    base_idx = to_np(icache).copy()
    base_kv = to_np(kcache).copy()
    dsa.paged_write_layer(bf16(new_idx, "cuda"), icache, bf16(new_kv, "cuda"), kcache,
                          i32(pt, "cuda"), d.seq_lens, i32(cu, "cuda"))
    torch.cuda.synchronize()
    exp_idx = oracle.paged_write(base_idx, bf16_to_f64(new_idx), 0, pt, wl.seq_lens, cu)
    exp_kv = oracle.paged_write(base_kv, bf16_to_f64(new_kv), 0, pt, wl.seq_lens, cu)
    assert np.array_equal(to_np(icache), exp_idx, equal_nan=True), "indexer cache differs"
    assert np.array_equal(to_np(kcache), exp_kv, equal_nan=True), "latent cache differs"
    # the rows of the two pages without a slot kept their poison; every other
    # chunk slot holds its row again
    pg = pt[seq, pos // wl.PS]
    ok = (pg >= 0) & (pg < P)
    assert (~ok).sum() >= 2 and not ok[t1] and not ok[t2]
    assert np.isnan(to_np(icache).reshape(-1, wl.D_idx)[slots[~ok]]).all()
    assert not np.isnan(to_np(kcache).reshape(-1, 576)[slots[ok]]).any()


def _rows(T, cu, n, seed):
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    for c in cu[1:-1]:
        rows.update({int(c) - 1, int(c)})
    rows.update(rng.choice(T, size=n, replace=False).tolist())
    return sorted(rows)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("path", [None, "per_query", 64, 256])
def test_extend_layers_config4_mixed_share(dsa, path):
    torch = torch_mod()
    kinds = ["full", "shared", "full", "shared"]
    wl = W.config(4, layers=4)
    b = wl.batches["extend"]
    cu = b.cu_q_lens
    T = b.T
    # the second full layer's indexer inputs: the same integer-valued
    # distributions, rearranged (negated queries, reversed head weights)
    qi = [b.q_idx, W.f32_to_bf16(-W.bf16_to_f32(b.q_idx))]
    ws = [b.w, np.ascontiguousarray(b.w[:, ::-1])]
    d = Dev(wl)
    new_idx, slots = _chunk_rows(wl.idx_cache, wl, cu)
    new_kv = [_chunk_rows(wl.kv_cache[i], wl, cu)[0] for i in range(4)]
    icaches = [_poisoned(wl.idx_cache.to_torch("cuda"), slots) for _ in range(2)]
    kcaches = [_poisoned(d.kv_cache[i], slots) for i in range(4)]
    qs = [bf16(b.q_mla[i], "cuda") for i in range(4)]
    log(f"extend layers {kinds}: path {path}, T={T}")
    outs, info = dsa.extend_layers(
        kinds, page_table=d.page_table, seq_lens=d.seq_lens, cu_q_lens=i32(cu, "cuda"),
        k=wl.k, max_q_len=int(np.diff(cu).max()), sm_scale=wl.sm_scale,
        q_idx=[bf16(x, "cuda") for x in qi], w=[torch.from_numpy(x.copy()).cuda() for x in ws],
        idx_cache=icaches, q=qs, kv_cache=kcaches,
        new_idx=[bf16(new_idx, "cuda")] * 2, new_kv=[bf16(x, "cuda") for x in new_kv],
        qb_candidates=(64, 256), path=path)
    torch.cuda.synchronize()
    log(f"  choices {info['choice']}, src slots {info['src_slot']}")
    assert info["src_slot"] == {0: 0, 1: 0, 2: 1, 3: 1}
    if path is None:
        assert all(c in (0, 64, 256) for c in info["choice"])
    else:
        assert info["choice"] == [0 if path == "per_query" else path] * 2
    rows = _rows(T, cu, 40, 7)
    icache64 = wl.idx_cache.f64_view()
    for slot in range(2):
        tk = info["topk"][slot].cpu().numpy()
        check_topk_rows_valid(tk, wl.seq_lens, cu, wl.k)
        exp = oracle.indexer_topk(bf16_to_f64(qi[slot]), ws[slot].astype(np.float64), icache64,
                                  wl.page_table, wl.seq_lens, cu, wl.k, rows=rows)
        # the layer loop asks for position order: the oracle's rows sorted
        srt = np.sort(np.where(exp[rows] >= 0, exp[rows].astype(np.int64), 1 << 40), axis=1)
        assert np.array_equal(tk[rows], np.where(srt == 1 << 40, -1, srt)), \
            f"slot {slot} top-k differs from the oracle"
        assert ((tk[:, 1:] > tk[:, :-1]) | (tk[:, 1:] < 0)).all(), "rows not in position order"
        for layer in (2 * slot, 2 * slot + 1):
            ref = oracle.sparse_mla(bf16_to_f64(b.q_mla[layer]), wl.kv_cache[layer].f64_view(),
                                    wl.page_table, wl.seq_lens, cu, exp, wl.sm_scale, wl.Dv,
                                    rows=rows)
            check_attention(to_np(outs[layer]), ref, rows=rows,
                            what=f"layer {layer} ({kinds[layer]}, slot {slot}, path {path})")
