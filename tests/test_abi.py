"""The C-ABI library: it loads, exports every declared symbol, and its host
validation rejects bad arguments before touching the GPU (no compute call
is made here)."""
import ctypes
import os

import numpy as np

import pytest

import sparse_attention_relu_amd as dsa
from sparse_attention_relu_amd import _lib


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_relu_amd import build

        build.build(verbose=False)
    return dsa.load()


def test_exports_every_declared_symbol(lib):
    declared = _lib.header_functions()
    assert len(declared) == 27
    assert "dsa_sparse_mla_decode_static" in declared
    assert "dsa_indexer_topk_ordered" in declared and "dsa_topk_position_order" in declared
    for name in declared:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"
    assert sorted(_lib.SIGNATURES) == declared


def test_status_strings(lib):
    assert dsa.status_string(0) == "ok"
    assert "workspace" in dsa.status_string(3)
    assert lib.dsa_abi_version() == 2


def _idx_call(lib, **kw):
    a = dict(q=1 << 12, w=1 << 12, cache=1 << 12, P=4, pt=1 << 12, sl=1 << 12, cu=1 << 12,
             T=2, S=1, H=32, D=128, PS=64, MP=4, k=16, mql=1, out=1 << 12, ws=None, wsb=0)
    a.update(kw)
    return lib.dsa_indexer_topk(a["q"], a["w"], a["cache"], a["P"], a["pt"], a["sl"], a["cu"],
                                a["T"], a["S"], a["H"], a["D"], a["PS"], a["MP"], a["k"],
                                a["mql"], a["out"], a["ws"], a["wsb"], None)


def test_indexer_validation(lib):
    assert _idx_call(lib, D=96) == _lib.DSA_ERR_UNSUPPORTED
    assert _idx_call(lib, k=0) == _lib.DSA_ERR_UNSUPPORTED
    assert _idx_call(lib, k=5000) == _lib.DSA_ERR_UNSUPPORTED
    assert _idx_call(lib, H=65) == _lib.DSA_ERR_UNSUPPORTED
    assert _idx_call(lib, PS=24) == _lib.DSA_ERR_UNSUPPORTED  # a load stages 16 rows of one page
    assert _idx_call(lib, T=-1) == _lib.DSA_ERR_INVALID_ARG
    assert _idx_call(lib, q=None) == _lib.DSA_ERR_INVALID_ARG
    assert _idx_call(lib, q=(1 << 12) + 2) == _lib.DSA_ERR_INVALID_ARG  # misaligned
    assert _idx_call(lib) == _lib.DSA_ERR_WORKSPACE  # no workspace given
    assert "workspace" in dsa.last_error()
    assert _idx_call(lib, T=0) == _lib.DSA_OK  # nothing to do: no launch
    need = dsa.indexer_topk_workspace(2, 1, 32, 128, 64, 4, 16, 1)
    assert need >= 2 * 4 * 64 * 4
    assert _idx_call(lib, ws=1 << 12, wsb=need - 1) == _lib.DSA_ERR_WORKSPACE


def test_ordered_entries_validation(lib):
    def ordered(order, **kw):
        a = dict(T=2, ws=None)
        a.update(kw)
        return lib.dsa_indexer_topk_ordered(1 << 12, 1 << 12, 1 << 12, 4, 1 << 12, 1 << 12,
                                            1 << 12, a["T"], 1, 32, 128, 64, 4, 16, 1, order,
                                            1 << 12, a["ws"], 0, None)

    assert ordered(2) == _lib.DSA_ERR_INVALID_ARG
    assert "order" in dsa.last_error()
    assert ordered(-1) == _lib.DSA_ERR_INVALID_ARG
    assert ordered(_lib.DSA_ORDER_POSITION) == _lib.DSA_ERR_WORKSPACE  # valid order, no workspace
    assert ordered(_lib.DSA_ORDER_SCORE, T=0) == _lib.DSA_OK
    fused = lib.dsa_indexer_topk_fused(1 << 12, 1 << 12, 1 << 12, 4, 1 << 12, 1 << 12, 1 << 12,
                                       2, 1, 32, 128, 64, 4, 16, 7, 1 << 12, None, 0, None)
    assert fused == _lib.DSA_ERR_INVALID_ARG
    with pytest.raises(ValueError):
        _lib._order("descending")
    # the row sort: k out of range, NULL pointers, nothing to do
    assert lib.dsa_topk_position_order(1 << 12, 1 << 12, 4, 0, None) == _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_position_order(1 << 12, 1 << 12, 4, 4097, None) == \
        _lib.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk_position_order(None, 1 << 12, 4, 16, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_position_order(1 << 12, 1 << 12, -1, 16, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_topk_position_order(None, None, 0, 16, None) == _lib.DSA_OK


def test_union_validation(lib):
    def call(**kw):
        a = dict(T=8, S=2, k=4, PS=64, MP=8, QB=4, u_max=16, ws=None, wsb=0, units=1 << 12,
                 member=1 << 12)
        a.update(kw)
        return lib.dsa_block_union(1 << 12, 1 << 12, 1 << 12, a["T"], a["S"], a["k"], a["PS"],
                                   a["MP"], a["QB"], a["u_max"], a["units"], 1 << 12,
                                   a["member"], a["ws"], a["wsb"], None)

    assert call(PS=128) == _lib.DSA_ERR_UNSUPPORTED
    assert call(QB=0) == _lib.DSA_ERR_UNSUPPORTED
    assert call(u_max=0) == _lib.DSA_ERR_UNSUPPORTED
    assert call(u_max=100000) == _lib.DSA_ERR_UNSUPPORTED
    assert call(S=64, MP=8192) == _lib.DSA_ERR_UNSUPPORTED
    assert call() == _lib.DSA_ERR_WORKSPACE
    assert call(units=None) == _lib.DSA_ERR_INVALID_ARG
    assert call(member=None) == _lib.DSA_ERR_WORKSPACE  # sizes only: membership is optional
    assert call(T=0) == _lib.DSA_OK


def test_mla_validation(lib):
    def dec(**kw):
        # k = 2048 over 2 rows is split into chunks, so a workspace is needed
        a = dict(rs=576, H=16, k=2048, T=2, q=1 << 12)
        a.update(kw)
        return lib.dsa_sparse_mla_decode(a["q"], 1 << 12, a["rs"], 8, 1 << 12, 1 << 12, 1 << 12,
                                         1 << 12, a["T"], 2, a["H"], a["k"], 64, 4, 0.1,
                                         1 << 12, None, 0, None)

    assert dec(rs=500) == _lib.DSA_ERR_INVALID_ARG
    assert dec(rs=580) == _lib.DSA_ERR_INVALID_ARG
    assert dec(H=0) == _lib.DSA_ERR_UNSUPPORTED
    assert dec(q=(1 << 12) + 8) == _lib.DSA_ERR_INVALID_ARG
    assert dec() == _lib.DSA_ERR_WORKSPACE
    assert dec(T=0) == _lib.DSA_OK

    def ext(**kw):
        a = dict(H=16, PS=64, QB=64, u_max=32)
        a.update(kw)
        return lib.dsa_sparse_mla_extend(1 << 12, 1 << 12, 576, 8, 1 << 12, 1 << 12, 1 << 12,
                                         1 << 12, 1 << 12, 1 << 12, 4, 2, a["H"], a["PS"], 4,
                                         a["QB"], a["u_max"], 0.1, 1 << 12, None, 0, None)

    assert ext(H=65) == _lib.DSA_ERR_UNSUPPORTED
    assert ext(PS=128) == _lib.DSA_ERR_UNSUPPORTED
    assert ext(QB=2048) == _lib.DSA_ERR_UNSUPPORTED
    assert ext(u_max=0) == _lib.DSA_ERR_INVALID_ARG


def test_decode_workspace_formula(lib):
    # partial (m, l, O) per (row, chunk, head)
    ws = dsa.sparse_mla_decode_workspace(8, 16, 2048)
    assert ws > 0 and ws % 256 == 0
    assert dsa.sparse_mla_decode_workspace(0, 16, 2048) == 0
    # a batch with one chunk per row (8192 rows of 2048 selections) writes its
    # output directly: no workspace
    assert dsa.sparse_mla_decode_workspace(8192, 16, 2048) == 0


def test_extend_attend_path(lib):
    """Host-side choice between the query-block and per-query extend paths:
    the long-context shape (8192 queries, unions of about 2000 of 2048
    pages, 62x the useful MFMA work) goes per query; unions of half the
    chunked-extend size, or tiny ones, keep the query block (at the full
    chunked-extend size, about 200 of 208 pages, the two paths measure
    within a few percent of each other)."""
    import numpy as np

    assert dsa.extend_attend_path(np.full(16, 100), 4096, 16, 2048, 64, 256, 832) == "qblock"
    assert dsa.extend_attend_path(np.full(32, 1986), 8192, 16, 2048, 64, 256, 2048) == \
        "per_query"
    assert dsa.extend_attend_path(np.full(64, 4), 4096, 16, 2048, 64, 64, 832) == "qblock"
    # counts beyond u_max are capped (the kernel walks at most u_max slots)
    a = dsa.extend_attend_path(np.full(16, 10 ** 6), 4096, 16, 2048, 64, 256, 208)
    assert a == dsa.extend_attend_path(np.full(16, 208), 4096, 16, 2048, 64, 256, 208)
    c = np.zeros(3, dtype=np.int32)
    assert lib.dsa_extend_attend_path(c.ctypes.data, 3, 100, 16, 2048, 64, 64, 8) == \
        -_lib.DSA_ERR_INVALID_ARG  # nQB != ceil(T / QB)
    assert lib.dsa_extend_attend_path(None, 2, 100, 16, 2048, 64, 64, 8) == \
        -_lib.DSA_ERR_INVALID_ARG
    with pytest.raises(dsa.DsaError):
        dsa.extend_attend_path(np.zeros(2), 100, 16, 0, 64, 64, 8)


def test_page_entry_validation(lib):
    def call(**kw):
        a = dict(T=2, S=1, H=32, D=128, PS=64, MP=4, kp=4, ws=None, wsb=0)
        a.update(kw)
        return lib.dsa_indexer_page_topk(1 << 12, 1 << 12, 1 << 12, 4, 1 << 12, 1 << 12, 1 << 12,
                                         a["T"], a["S"], a["H"], a["D"], a["PS"], a["MP"],
                                         a["kp"], 1, 1 << 12, a["ws"], a["wsb"], None)

    assert call(kp=0) == _lib.DSA_ERR_UNSUPPORTED
    assert call(kp=5000) == _lib.DSA_ERR_UNSUPPORTED
    assert call(PS=128, MP=2) == _lib.DSA_ERR_UNSUPPORTED  # one 16-lane group pools a page
    assert call(PS=24) == _lib.DSA_ERR_UNSUPPORTED
    assert call() == _lib.DSA_ERR_WORKSPACE
    assert call(T=0) == _lib.DSA_OK
    need = dsa.indexer_page_topk_workspace(2, 1, 32, 128, 64, 4, 4, 1)
    assert need >= dsa.indexer_topk_workspace(2, 1, 32, 128, 64, 4, 4, 1) + 2 * 4 * 4
    assert lib.dsa_page_tokens(1 << 12, 2, 0, 64, 1 << 12, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_page_tokens(1 << 12, 2, 2048, 64, 1 << 12, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_page_tokens(None, 2, 4, 64, 1 << 12, None) == _lib.DSA_ERR_INVALID_ARG
    assert lib.dsa_page_tokens(1 << 12, 0, 4, 64, 1 << 12, None) == _lib.DSA_OK


def test_paged_write_validation(lib):
    def call(**kw):
        a = dict(ss=576, cols=512, col0=0, rs=576, T=2, S=1, PS=64, MP=4, src=1 << 12)
        a.update(kw)
        return lib.dsa_paged_write(a["src"], a["ss"], a["cols"], a["col0"], 1 << 12, a["rs"], 4,
                                   1 << 12, 1 << 12, 1 << 12, a["T"], a["S"], a["PS"], a["MP"],
                                   None)

    assert call(cols=12) == _lib.DSA_ERR_INVALID_ARG
    assert call(col0=4) == _lib.DSA_ERR_INVALID_ARG
    assert call(col0=512, cols=128) == _lib.DSA_ERR_INVALID_ARG  # past the row
    assert call(ss=256) == _lib.DSA_ERR_INVALID_ARG  # src rows shorter than cols
    assert call(src=(1 << 12) + 2) == _lib.DSA_ERR_INVALID_ARG  # misaligned
    assert call(src=None) == _lib.DSA_ERR_INVALID_ARG
    assert call(T=0) == _lib.DSA_OK


def test_index_share_map(lib):
    """Full layers own consecutive slots; a shared layer uses the nearest
    preceding full layer's slot; a leading shared layer is an error."""
    full, src, n = dsa.index_share_map(["full", "shared", "shared", "full", "shared"])
    assert n == 2 and full == {0: 0, 3: 1}
    assert src == {0: 0, 1: 0, 2: 0, 3: 1, 4: 1}
    full, src, n = dsa.index_share_map(["full"] * 3)
    assert n == 3 and full == {0: 0, 1: 1, 2: 2} and src == {0: 0, 1: 1, 2: 2}
    assert dsa.index_share_map([]) == ({}, {}, 0)
    with pytest.raises(dsa.DsaError):
        dsa.index_share_map(["shared", "full"])
    with pytest.raises(ValueError):
        dsa.index_share_map(["full", "dense"])


def test_static_decode_host_checks(lib):
    """The allocation-free decode refuses, on the host and before any HIP
    call, an unsupported head count and a batch whose partials exceed its
    32 MiB static scratch."""
    p = 1 << 12
    args = lambda T, H, k: (p, p, 576, 4, p, p, p, p, T, 1, H, k, 64, 4, 0.1, p, None)
    assert lib.dsa_sparse_mla_decode_static(*args(2, 0, 16)) == 2
    assert lib.dsa_sparse_mla_decode_static(*args(64, 64, 65536)) == 2
    assert "static scratch" in dsa.last_error()
    assert lib.dsa_sparse_mla_decode_static(*args(0, 16, 16)) == 0  # empty batch: nothing to do


def test_extend_attend_plan_picks_cheapest(lib):
    """Host logic: the per-query path for saturated unions at the chunked
    size; a query block when unions are small, the larger block when its
    union is smaller per row."""
    T, H, k, PS = 4096, 16, 2048, 64
    sat = {64: np.full(64, 208), 256: np.full(16, 208)}
    assert dsa.extend_attend_plan(sat, T, H, k, PS, 832) == 0
    small = {64: np.full(64, 4), 256: np.full(16, 4)}
    assert dsa.extend_attend_plan(small, T, H, k, PS, 832) == 64  # a tie keeps the first
    small[256] = np.full(16, 3)
    assert dsa.extend_attend_plan(small, T, H, k, PS, 832) == 256
    assert dsa.extend_attend_plan({}, T, H, k, PS, 832) == 0
    with pytest.raises(dsa.DsaError):
        dsa.extend_attend_plan({0: np.zeros(1)}, T, H, k, PS, 832)
