"""The decode layer (indexer top-k, then sparse MLA decode) and the extend
attention captured as a HIP graph (torch.cuda.CUDAGraph) and replayed: every
replay, with eager work and synchronisations between replays, gives exactly
the eager results. The library records no memset and allocates nothing, so
its launches are capturable as they are."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import Dev, log, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_relu_amd as m

    m.load()
    return m


def _replays_match(step, outs, n=4):
    """Eager results of `step`, then n replays of its graph compared with them."""
    torch = torch_mod()
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(n):
        for o in outs:
            o.zero_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("cid", [1, 2])
def test_decode_layer_graph_replay(dsa, cid):
    torch = torch_mod()
    wl = W.config(cid)
    b = wl.batches["decode"]
    d = Dev(wl)
    bt = d.batch("decode")
    T, k, H = b.T, wl.k, wl.H_mla
    topk = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    ws_i = torch.empty(max(1, dsa.indexer_topk_workspace(T, wl.S, wl.H_idx, wl.D_idx, wl.PS,
                                                         wl.MP, k, 1)),
                       dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(max(1, dsa.sparse_mla_decode_workspace(T, H, k)), dtype=torch.uint8,
                       device="cuda")

    def step():
        dsa.indexer_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens, bt["cu"],
                         k, 1, out=topk, workspace=ws_i)
        dsa.sparse_mla_decode(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"], topk,
                              wl.sm_scale, out=out, workspace=ws_d)

    log(f"config {cid}: decode layer, graph replays")
    _replays_match(step, [topk, out])


def test_extend_attention_graph_replay(dsa):
    """The tiny workload's extend batch: indexer, union and query-block attention."""
    torch = torch_mod()
    wl = W.config(1)
    b = wl.batches["extend"]
    d = Dev(wl)
    bt = d.batch("extend")
    T, k, H, QB = b.T, wl.k, wl.H_mla, 16
    mql = int(np.diff(b.cu_q_lens).max())
    nqb = (T + QB - 1) // QB
    topk = torch.empty((T, k), dtype=torch.int32, device="cuda")
    units = torch.empty((nqb, wl.u_max), dtype=torch.int32, device="cuda")
    counts = torch.empty((nqb,), dtype=torch.int32, device="cuda")
    member = torch.empty((nqb, wl.u_max, QB), dtype=torch.uint64, device="cuda")
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    ws_i = torch.empty(max(1, dsa.indexer_topk_workspace(T, wl.S, wl.H_idx, wl.D_idx, wl.PS,
                                                         wl.MP, k, mql)),
                       dtype=torch.uint8, device="cuda")
    ws_u = torch.empty(max(1, dsa.block_union_workspace(T, wl.S, wl.MP, QB, wl.u_max)),
                       dtype=torch.uint8, device="cuda")

    def step():
        dsa.indexer_topk(bt["q_idx"], bt["w"], d.idx_cache, d.page_table, d.seq_lens, bt["cu"],
                         k, mql, out=topk, workspace=ws_i)
        dsa.block_union(topk, d.seq_lens, bt["cu"], wl.PS, wl.MP, QB, wl.u_max,
                        out=(units, counts, member), workspace=ws_u)
        dsa.sparse_mla_extend(bt["q"], d.kv_cache[0], d.page_table, d.seq_lens, bt["cu"], units,
                              counts, member, QB, wl.sm_scale, out=out)

    log("config 1: extend layer, graph replays")
    _replays_match(step, [topk, units, counts, member, out])
