"""ctypes binding of libdsa.so (include/dsa.h).

Argument marshalling only: every function checks tensor dtypes, shapes and
devices, allocates outputs and workspace with torch (device memory is the
only thing torch provides here), and hands raw pointers plus the current
HIP stream to the C entry point of the same name. There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "dsa.h")

DSA_OK = 0
DSA_ERR_INVALID_ARG = 1
DSA_ERR_UNSUPPORTED = 2
DSA_ERR_WORKSPACE = 3
DSA_ERR_HIP = 4

_c_int, _c_size, _c_float, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

# name -> (restype, argtypes); must match include/dsa.h
SIGNATURES = {
    "dsa_status_string": (ctypes.c_char_p, [_c_int]),
    "dsa_last_error": (ctypes.c_char_p, []),
    "dsa_abi_version": (_c_int, []),
    "dsa_indexer_topk_workspace": (_c_size, [_c_int] * 8),
    "dsa_indexer_topk": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 8
                         + [_vp, _vp, _c_size, _vp]),
    "dsa_indexer_topk_fused_workspace": (_c_size, [_c_int] * 7),
    "dsa_indexer_topk_ordered": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 9
                                 + [_vp, _vp, _c_size, _vp]),
    "dsa_topk_position_order": (_c_int, [_vp, _vp, _c_int, _c_int, _vp]),
    "dsa_indexer_topk_fused": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 8
                               + [_vp, _vp, _c_size, _vp]),
    "dsa_block_union_workspace": (_c_size, [_c_int] * 5),
    "dsa_block_union": (_c_int, [_vp, _vp, _vp] + [_c_int] * 7 + [_vp, _vp, _vp, _vp, _c_size,
                                                                  _vp]),
    "dsa_sparse_mla_decode_workspace": (_c_size, [_c_int] * 3),
    "dsa_sparse_mla_decode": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp]
                              + [_c_int] * 6 + [_c_float, _vp, _vp, _c_size, _vp]),
    "dsa_sparse_mla_extend_workspace": (_c_size, [_c_int] * 4),
    "dsa_extend_attend_path": (_c_int, [_vp] + [_c_int] * 7),
    "dsa_extend_attend_plan": (_c_int, [_c_int, _vp, _vp] + [_c_int] * 5),
    "dsa_index_share_map": (_c_int, [_vp, _c_int, _vp, _vp]),
    "dsa_indexer_page_topk_workspace": (_c_size, [_c_int] * 8),
    "dsa_indexer_page_topk": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 8
                              + [_vp, _vp, _c_size, _vp]),
    "dsa_page_tokens": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "dsa_paged_write": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp]
                        + [_c_int] * 4 + [_vp]),
    "dsa_paged_write_layer": (_c_int, [_vp, _c_int, _vp, _vp, _c_int, _vp, _c_int, _c_int,
                                       _vp, _vp, _vp] + [_c_int] * 4 + [_vp]),
    "dsa_sparse_mla_decode_static": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp]
                                     + [_c_int] * 6 + [_c_float, _vp, _vp]),
    "dsa_sparse_mla_decode_pages": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp]
                                    + [_c_int] * 6 + [_c_float, _vp, _vp, _c_size, _vp]),
    "dsa_profile_enable": (_c_int, [_c_int]),
    "dsa_profile_read": (_c_int, [_c_int, ctypes.c_char_p, _c_int, _vp, _vp, _vp]),
    "dsa_sparse_mla_extend": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp]
                              + [_c_int] * 7 + [_c_float, _vp, _vp, _c_size, _vp]),
}


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {status_string(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so once; raises ImportError when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with "
                          "`python -m sparse_attention_relu_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/dsa.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def status_string(status: int) -> str:
    return load().dsa_status_string(status).decode()


def last_error() -> str:
    return load().dsa_last_error().decode()


def _check(fn: str, status: int):
    if status != DSA_OK:
        raise DsaError(fn, status, last_error())


# ----------------------------------------------------------------------------
# torch marshalling helpers
# ----------------------------------------------------------------------------
def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t, name, dtype, ndim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _alloc_stream(stream):
    """The stream a tensor the binding allocates must belong to: memory
    from torch's caching allocator is tied to the stream it is allocated on,
    so a buffer that the library uses on another stream is allocated on that
    stream (its memory is then not reused before that stream's work)."""
    torch = _torch()
    if stream is None or stream == torch.cuda.current_stream():
        return None
    return stream


def _empty(shape, dtype, device, stream=None):
    torch = _torch()
    s = _alloc_stream(stream)
    if s is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(s):
        return torch.empty(shape, dtype=dtype, device=device)


def _workspace(nbytes: int, device, workspace=None, stream=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")
        return workspace
    return _empty(nbytes, torch.uint8, device, stream)


def _ragged(page_table, seq_lens, cu_q_lens, device):
    torch = _torch()
    _need(page_table, "page_table", torch.int32, 2, device)
    _need(seq_lens, "seq_lens", torch.int32, 1, device)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1, device)
    S = seq_lens.shape[0]
    if page_table.shape[0] != S or cu_q_lens.shape[0] != S + 1:
        raise ValueError("page_table [S, MP], seq_lens [S], cu_q_lens [S+1] disagree on S")
    return S, page_table.shape[1]


# ----------------------------------------------------------------------------
# Kernel timing
# ----------------------------------------------------------------------------
def profile_enable(on: bool = True) -> None:
    """Start (and clear) or stop per-kernel event timing in the library."""
    _check("dsa_profile_enable", load().dsa_profile_enable(1 if on else 0))


def profile_read(max_kernels: int = 32):
    """{kernel name: (launches, total_ms)} of the launches since enabling."""
    name_len = 64
    names = ctypes.create_string_buffer(max_kernels * name_len)
    launches = (ctypes.c_int * max_kernels)()
    total = (ctypes.c_double * max_kernels)()
    n = ctypes.c_int(0)
    st = load().dsa_profile_read(max_kernels, names, name_len, ctypes.addressof(launches),
                                 ctypes.addressof(total), ctypes.addressof(n))
    _check("dsa_profile_read", st)
    raw = names.raw
    out = {}
    for i in range(n.value):
        nm = raw[i * name_len:(i + 1) * name_len].split(b"\0", 1)[0].decode()
        out[nm] = (launches[i], total[i])
    return out


# ----------------------------------------------------------------------------
# Entry points
# ----------------------------------------------------------------------------
def indexer_topk_workspace(T, S, H, D, PS, MP, k, max_q_len) -> int:
    return load().dsa_indexer_topk_workspace(T, S, H, D, PS, MP, k, max_q_len)


DSA_ORDER_SCORE, DSA_ORDER_POSITION = 0, 1
_ORDERS = {"score": DSA_ORDER_SCORE, "position": DSA_ORDER_POSITION}


def _order(order) -> int:
    if order not in _ORDERS:
        raise ValueError(f"order {order!r} is neither 'score' nor 'position'")
    return _ORDERS[order]


def indexer_topk(q_idx, w, idx_cache, page_table, seq_lens, cu_q_lens, k: int,
                 max_q_len: int, out=None, workspace=None, stream=None, order="score"):
    """Exact lightning-indexer top-k -> int32 [T, k] (dsa_indexer_topk;
    order="position": the same positions ascending, dsa_indexer_topk_ordered)."""
    ordv = _order(order)
    torch = _torch()
    dev = q_idx.device
    _need(q_idx, "q_idx", torch.bfloat16, 3, dev)
    _need(w, "w", torch.float32, 2, dev)
    _need(idx_cache, "idx_cache", torch.bfloat16, 3, dev)
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T, H, D = q_idx.shape
    P, PS, Dc = idx_cache.shape
    if Dc != D or tuple(w.shape) != (T, H):
        raise ValueError("q_idx [T,H,D], w [T,H], idx_cache [P,PS,D] disagree")
    if out is None:
        out = _empty((T, k), torch.int32, dev, stream)
    _need(out, "out", torch.int32, 2, dev)
    nbytes = indexer_topk_workspace(T, S, H, D, PS, MP, k, max_q_len)
    ws = _workspace(nbytes, dev, workspace, stream)
    if ordv == DSA_ORDER_SCORE:
        st = load().dsa_indexer_topk(_ptr(q_idx), _ptr(w), _ptr(idx_cache), P, _ptr(page_table),
                                     _ptr(seq_lens), _ptr(cu_q_lens), T, S, H, D, PS, MP, k,
                                     max_q_len, _ptr(out), _ptr(ws), nbytes, _stream(stream))
        _check("dsa_indexer_topk", st)
    else:
        st = load().dsa_indexer_topk_ordered(_ptr(q_idx), _ptr(w), _ptr(idx_cache), P,
                                             _ptr(page_table), _ptr(seq_lens), _ptr(cu_q_lens),
                                             T, S, H, D, PS, MP, k, max_q_len, ordv, _ptr(out),
                                             _ptr(ws), nbytes, _stream(stream))
        _check("dsa_indexer_topk_ordered", st)
    return out


def topk_position_order(topk, out=None, stream=None):
    """Each row of a top-k table in ascending position order, -1 entries
    last -> int32 [T, k] (dsa_topk_position_order; out may be topk)."""
    torch = _torch()
    dev = topk.device
    _need(topk, "topk", torch.int32, 2, dev)
    T, k = topk.shape
    if out is None:
        out = _empty((T, k), torch.int32, dev, stream)
    _need(out, "out", torch.int32, 2, dev)
    if tuple(out.shape) != (T, k):
        raise ValueError(f"out {tuple(out.shape)} != {(T, k)}")
    st = load().dsa_topk_position_order(_ptr(topk), _ptr(out), T, k, _stream(stream))
    _check("dsa_topk_position_order", st)
    return out


def indexer_topk_fused_workspace(T, S, H, D, PS, MP, k) -> int:
    return load().dsa_indexer_topk_fused_workspace(T, S, H, D, PS, MP, k)


def indexer_topk_fused(q_idx, w, idx_cache, page_table, seq_lens, cu_q_lens, k: int, out=None,
                       workspace=None, stream=None, order="score"):
    """Exact lightning-indexer top-k without the score matrix -> int32
    [T, k] (dsa_indexer_topk_fused); the same result as indexer_topk."""
    ordv = _order(order)
    torch = _torch()
    dev = q_idx.device
    _need(q_idx, "q_idx", torch.bfloat16, 3, dev)
    _need(w, "w", torch.float32, 2, dev)
    _need(idx_cache, "idx_cache", torch.bfloat16, 3, dev)
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T, H, D = q_idx.shape
    P, PS, Dc = idx_cache.shape
    if Dc != D or tuple(w.shape) != (T, H):
        raise ValueError("q_idx [T,H,D], w [T,H], idx_cache [P,PS,D] disagree")
    if out is None:
        out = _empty((T, k), torch.int32, dev, stream)
    _need(out, "out", torch.int32, 2, dev)
    nbytes = indexer_topk_fused_workspace(T, S, H, D, PS, MP, k)
    ws = _workspace(nbytes, dev, workspace, stream)
    st = load().dsa_indexer_topk_fused(_ptr(q_idx), _ptr(w), _ptr(idx_cache), P,
                                       _ptr(page_table), _ptr(seq_lens), _ptr(cu_q_lens), T, S,
                                       H, D, PS, MP, k, ordv, _ptr(out), _ptr(ws), nbytes,
                                       _stream(stream))
    _check("dsa_indexer_topk_fused", st)
    return out


def indexer_page_topk_workspace(T, S, H, D, PS, MP, k_pages, max_q_len) -> int:
    return load().dsa_indexer_page_topk_workspace(T, S, H, D, PS, MP, k_pages, max_q_len)


def indexer_page_topk(q_idx, w, idx_cache, page_table, seq_lens, cu_q_lens, k_pages: int,
                      max_q_len: int, out=None, workspace=None, stream=None):
    """Exact page-level indexer top-k -> int32 [T, k_pages] seq-local page
    ids (dsa_indexer_page_topk)."""
    torch = _torch()
    dev = q_idx.device
    _need(q_idx, "q_idx", torch.bfloat16, 3, dev)
    _need(w, "w", torch.float32, 2, dev)
    _need(idx_cache, "idx_cache", torch.bfloat16, 3, dev)
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T, H, D = q_idx.shape
    P, PS, Dc = idx_cache.shape
    if Dc != D or tuple(w.shape) != (T, H):
        raise ValueError("q_idx [T,H,D], w [T,H], idx_cache [P,PS,D] disagree")
    if out is None:
        out = _empty((T, k_pages), torch.int32, dev, stream)
    _need(out, "out", torch.int32, 2, dev)
    nbytes = indexer_page_topk_workspace(T, S, H, D, PS, MP, k_pages, max_q_len)
    ws = _workspace(nbytes, dev, workspace, stream)
    st = load().dsa_indexer_page_topk(_ptr(q_idx), _ptr(w), _ptr(idx_cache), P,
                                      _ptr(page_table), _ptr(seq_lens), _ptr(cu_q_lens), T, S,
                                      H, D, PS, MP, k_pages, max_q_len, _ptr(out), _ptr(ws),
                                      nbytes, _stream(stream))
    _check("dsa_indexer_page_topk", st)
    return out


def page_tokens(pages, PS: int, out=None, stream=None):
    """Positions of selected pages -> int32 [T, k_pages * PS] (dsa_page_tokens)."""
    torch = _torch()
    dev = pages.device
    _need(pages, "pages", torch.int32, 2, dev)
    T, kp = pages.shape
    if out is None:
        out = _empty((T, kp * PS), torch.int32, dev, stream)
    _need(out, "out", torch.int32, 2, dev)
    st = load().dsa_page_tokens(_ptr(pages), T, kp, PS, _ptr(out), _stream(stream))
    _check("dsa_page_tokens", st)
    return out


def paged_write(src, cache, page_table, seq_lens, cu_q_lens, col0: int = 0, stream=None):
    """Write row t of src (bf16 [T, cols], unit column stride) into the cache
    slot of its sequence position, columns col0 .. col0 + cols - 1
    (dsa_paged_write). The cache tensor is updated in place and returned."""
    torch = _torch()
    dev = cache.device
    _need(cache, "cache", torch.bfloat16, 3, dev)
    if src.dtype != torch.bfloat16 or src.dim() != 2 or src.device != dev or src.stride(1) != 1:
        raise ValueError("src must be a bf16 [T, cols] tensor with unit column stride on "
                         "the cache's device")
    if not cache.is_contiguous():
        raise ValueError("cache must be contiguous")
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T, cols = src.shape
    P, PS, rs = cache.shape
    st = load().dsa_paged_write(_ptr(src), src.stride(0), cols, col0, _ptr(cache), rs, P,
                                _ptr(page_table), _ptr(seq_lens), _ptr(cu_q_lens), T, S, PS, MP,
                                _stream(stream))
    _check("dsa_paged_write", st)
    return cache


def paged_write_layer(idx_src, idx_cache, kv_src, kv_cache, page_table, seq_lens, cu_q_lens,
                      stream=None):
    """Write a layer's new tokens into its indexer-key cache and its latent
    cache with one launch (dsa_paged_write_layer). idx_src bf16 [T, D] and
    kv_src bf16 [T, cols] are dense; either (with its cache) may be None. The
    caches are updated in place."""
    torch = _torch()
    if idx_src is None and kv_src is None:
        raise ValueError("nothing to write: idx_src and kv_src are both None")
    ref = idx_cache if idx_src is not None else kv_cache
    dev = ref.device
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T = (idx_src if idx_src is not None else kv_src).shape[0]
    D, P, PS, cols, rs = 0, None, None, 0, 0
    if idx_src is not None:
        _need(idx_src, "idx_src", torch.bfloat16, 2, dev)
        _need(idx_cache, "idx_cache", torch.bfloat16, 3, dev)
        P, PS, D = idx_cache.shape
        if idx_src.shape[1] != D:
            raise ValueError("idx_src [T, D] and idx_cache [P, PS, D] disagree on D")
    if kv_src is not None:
        _need(kv_src, "kv_src", torch.bfloat16, 2, dev)
        _need(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
        P2, PS2, rs = kv_cache.shape
        if P is not None and (P2, PS2) != (P, PS):
            raise ValueError("the two caches must have the same pages")
        P, PS = P2, PS2
        cols = kv_src.shape[1]
        if kv_src.shape[0] != T:
            raise ValueError("idx_src and kv_src disagree on T")
    st = load().dsa_paged_write_layer(_ptr(idx_src), D, _ptr(idx_cache) if idx_src is not None
                                      else None, _ptr(kv_src), cols,
                                      _ptr(kv_cache) if kv_src is not None else None, rs, P,
                                      _ptr(page_table), _ptr(seq_lens), _ptr(cu_q_lens), T, S, PS,
                                      MP, _stream(stream))
    _check("dsa_paged_write_layer", st)


def block_union_workspace(T, S, MP, QB, u_max) -> int:
    return load().dsa_block_union_workspace(T, S, MP, QB, u_max)


def block_union(topk, seq_lens, cu_q_lens, PS: int, MP: int, QB: int, u_max: int,
                out=None, workspace=None, stream=None, member: bool = True):
    """Query-block union tables -> (units [nQB,u_max] i32, counts [nQB] i32,
    member [nQB,u_max,QB] u64) (dsa_block_union). member=False writes units
    and counts only and returns None for the membership table."""
    torch = _torch()
    dev = topk.device
    _need(topk, "topk", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1, dev)
    T, k = topk.shape
    S = seq_lens.shape[0]
    nqb = (T + QB - 1) // QB
    if out is None:
        out = (_empty((nqb, u_max), torch.int32, dev, stream),
               _empty((nqb,), torch.int32, dev, stream),
               _empty((nqb, u_max, QB), torch.uint64, dev, stream) if member else None)
    units, counts, mb = out
    _need(units, "units", torch.int32, 2, dev)
    _need(counts, "counts", torch.int32, 1, dev)
    if tuple(units.shape) != (nqb, u_max) or tuple(counts.shape) != (nqb,):
        raise ValueError(f"units {tuple(units.shape)} / counts {tuple(counts.shape)} do not "
                         f"match nQB={nqb}, u_max={u_max}")
    if not member:
        mb = None
    else:
        _need(mb, "member", torch.uint64, 3, dev)
        if tuple(mb.shape) != (nqb, u_max, QB):
            raise ValueError(f"member {tuple(mb.shape)} != {(nqb, u_max, QB)}")
    nbytes = block_union_workspace(T, S, MP, QB, u_max)
    ws = _workspace(nbytes, dev, workspace, stream)
    st = load().dsa_block_union(_ptr(topk), _ptr(seq_lens), _ptr(cu_q_lens), T, S, k, PS, MP, QB,
                                u_max, _ptr(units), _ptr(counts), _ptr(mb), _ptr(ws), nbytes,
                                _stream(stream))
    _check("dsa_block_union", st)
    return units, counts, mb


def _mla_common(q, kv_cache, page_table, seq_lens, cu_q_lens):
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, 3, dev)
    _need(kv_cache, "kv_cache", torch.bfloat16, 3, dev)
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T, H, Dk = q.shape
    if Dk != 576:
        raise ValueError(f"q last dim must be 576, got {Dk}")
    P, PS, row_stride = kv_cache.shape
    return dev, S, MP, T, H, P, PS, row_stride


def extend_attend_path(blk_counts, T: int, H: int, k: int, PS: int, QB: int,
                       u_max: int) -> str:
    """"qblock" or "per_query": the faster token-exact extend attention for
    a batch whose block unions are built (blk_counts: the union sizes, any
    array or tensor; a device tensor is copied to the host)."""
    import numpy as np

    if hasattr(blk_counts, "detach"):
        blk_counts = blk_counts.detach().cpu().numpy()
    c = np.ascontiguousarray(blk_counts, dtype=np.int32)
    r = load().dsa_extend_attend_path(c.ctypes.data, int(c.size), T, H, k, PS, QB, u_max)
    if r < 0:
        raise DsaError("dsa_extend_attend_path", -r, last_error())
    return "per_query" if r == 1 else "qblock"


def extend_attend_plan(counts_by_qb, T: int, H: int, k: int, PS: int, u_max: int) -> int:
    """The extend attention to run (dsa_extend_attend_plan): the chosen QB
    among the candidates, or 0 for the per-query path. counts_by_qb maps
    each candidate QB to its blk_counts (any array or tensor; a device
    tensor is copied to the host)."""
    import numpy as np

    qbs = [int(q) for q in counts_by_qb]
    arrs = []
    for q in qbs:
        c = counts_by_qb[q]
        if hasattr(c, "detach"):
            c = c.detach().cpu().numpy()
        arrs.append(np.ascontiguousarray(c, dtype=np.int32))
    qb_arr = np.asarray(qbs if qbs else [0], dtype=np.int32)
    ptrs = (ctypes.c_void_p * max(1, len(arrs)))(*[a.ctypes.data for a in arrs])
    r = load().dsa_extend_attend_plan(len(qbs), qb_arr.ctypes.data, ctypes.addressof(ptrs), T, H,
                                      k, PS, u_max)
    if r < 0:
        raise DsaError("dsa_extend_attend_plan", -r, last_error())
    return int(r)


def index_share_map(indexer_types):
    """IndexShare layer mapping (dsa_index_share_map). indexer_types lists
    "full" or "shared" per layer. Returns (full_slot, src_slot, num_full):
    full_slot maps each full layer to the slot it owns, src_slot maps every
    layer to the slot whose top-k it attends with."""
    import numpy as np

    kinds = []
    for i, kind in enumerate(indexer_types):
        if kind not in ("full", "shared"):
            raise ValueError(f"unknown indexer type {kind!r} at layer {i}")
        kinds.append(1 if kind == "full" else 0)
    n = len(kinds)
    lf = np.asarray(kinds, dtype=np.int32)
    fs = np.empty(max(n, 1), dtype=np.int32)
    ss = np.empty(max(n, 1), dtype=np.int32)
    r = load().dsa_index_share_map(lf.ctypes.data, n, fs.ctypes.data, ss.ctypes.data)
    if r < 0:
        raise DsaError("dsa_index_share_map", -r, last_error())
    full_slot = {i: int(fs[i]) for i in range(n) if kinds[i] == 1}
    src_slot = {i: int(ss[i]) for i in range(n)}
    return full_slot, src_slot, int(r)


def sparse_mla_decode_workspace(T, H, k) -> int:
    return load().dsa_sparse_mla_decode_workspace(T, H, k)


def sparse_mla_decode(q, kv_cache, page_table, seq_lens, cu_q_lens, topk, sm_scale: float,
                      out=None, workspace=None, stream=None):
    """Sparse absorbed MLA over each row's selection -> bf16 [T, H, 512]."""
    torch = _torch()
    dev, S, MP, T, H, P, PS, rs = _mla_common(q, kv_cache, page_table, seq_lens, cu_q_lens)
    _need(topk, "topk", torch.int32, 2, dev)
    if topk.shape[0] != T:
        raise ValueError("topk rows must match q rows")
    k = topk.shape[1]
    if out is None:
        out = _empty((T, H, 512), torch.bfloat16, dev, stream)
    nbytes = sparse_mla_decode_workspace(T, H, k)
    ws = _workspace(nbytes, dev, workspace, stream)
    st = load().dsa_sparse_mla_decode(_ptr(q), _ptr(kv_cache), rs, P, _ptr(page_table),
                                      _ptr(seq_lens), _ptr(cu_q_lens), _ptr(topk), T, S, H, k,
                                      PS, MP, float(sm_scale), _ptr(out), _ptr(ws), nbytes,
                                      _stream(stream))
    _check("dsa_sparse_mla_decode", st)
    return out


def sparse_mla_decode_static(q, kv_cache, page_table, seq_lens, cu_q_lens, topk,
                             sm_scale: float, out=None, stream=None):
    """sparse_mla_decode with the library's static per-GPU scratch instead of
    a workspace (dsa_sparse_mla_decode_static): nothing is allocated for the
    call apart from `out` when it is not given."""
    torch = _torch()
    dev, S, MP, T, H, P, PS, rs = _mla_common(q, kv_cache, page_table, seq_lens, cu_q_lens)
    _need(topk, "topk", torch.int32, 2, dev)
    if topk.shape[0] != T:
        raise ValueError("topk rows must match q rows")
    k = topk.shape[1]
    if out is None:
        out = _empty((T, H, 512), torch.bfloat16, dev, stream)
    _need(out, "out", torch.bfloat16, 3, dev)
    st = load().dsa_sparse_mla_decode_static(_ptr(q), _ptr(kv_cache), rs, P, _ptr(page_table),
                                             _ptr(seq_lens), _ptr(cu_q_lens), _ptr(topk), T, S,
                                             H, k, PS, MP, float(sm_scale), _ptr(out),
                                             _stream(stream))
    _check("dsa_sparse_mla_decode_static", st)
    return out


def sparse_mla_decode_pages(q, kv_cache, page_table, seq_lens, cu_q_lens, pages,
                            sm_scale: float, out=None, workspace=None, stream=None):
    """Sparse absorbed MLA over every valid position of each row's selected
    pages -> bf16 [T, H, 512] (dsa_sparse_mla_decode_pages)."""
    torch = _torch()
    dev, S, MP, T, H, P, PS, rs = _mla_common(q, kv_cache, page_table, seq_lens, cu_q_lens)
    _need(pages, "pages", torch.int32, 2, dev)
    if pages.shape[0] != T:
        raise ValueError("pages rows must match q rows")
    kp = pages.shape[1]
    if out is None:
        out = _empty((T, H, 512), torch.bfloat16, dev, stream)
    nbytes = sparse_mla_decode_workspace(T, H, kp * PS)
    ws = _workspace(nbytes, dev, workspace, stream)
    st = load().dsa_sparse_mla_decode_pages(_ptr(q), _ptr(kv_cache), rs, P, _ptr(page_table),
                                            _ptr(seq_lens), _ptr(cu_q_lens), _ptr(pages), T, S,
                                            H, kp, PS, MP, float(sm_scale), _ptr(out), _ptr(ws),
                                            nbytes, _stream(stream))
    _check("dsa_sparse_mla_decode_pages", st)
    return out


def sparse_mla_extend_workspace(T, H, QB, u_max) -> int:
    return load().dsa_sparse_mla_extend_workspace(T, H, QB, u_max)


def sparse_mla_extend(q, kv_cache, page_table, seq_lens, cu_q_lens, units, counts, member,
                      QB: int, sm_scale: float, out=None, workspace=None, stream=None):
    """Query-block sparse absorbed MLA -> bf16 [T, H, 512]."""
    torch = _torch()
    dev, S, MP, T, H, P, PS, rs = _mla_common(q, kv_cache, page_table, seq_lens, cu_q_lens)
    _need(units, "blk_units", torch.int32, 2, dev)
    _need(counts, "blk_counts", torch.int32, 1, dev)
    _need(member, "blk_member", torch.uint64, 3, dev)
    nqb, u_max = units.shape
    if nqb != (T + QB - 1) // QB or tuple(member.shape) != (nqb, u_max, QB):
        raise ValueError("union tables do not match (T, QB)")
    if out is None:
        out = _empty((T, H, 512), torch.bfloat16, dev, stream)
    nbytes = sparse_mla_extend_workspace(T, H, QB, u_max)
    ws = _workspace(nbytes, dev, workspace, stream)
    st = load().dsa_sparse_mla_extend(_ptr(q), _ptr(kv_cache), rs, P, _ptr(page_table),
                                      _ptr(seq_lens), _ptr(cu_q_lens), _ptr(units),
                                      _ptr(counts), _ptr(member), T, S, H, PS, MP, QB, u_max,
                                      float(sm_scale), _ptr(out), _ptr(ws) if ws is not None
                                      else None, nbytes, _stream(stream))
    _check("dsa_sparse_mla_extend", st)
    return out


# ----------------------------------------------------------------------------
# Layer runner (model-loop glue)
# ----------------------------------------------------------------------------
def extend_layers(indexer_types, *, page_table, seq_lens, cu_q_lens, k: int, max_q_len: int,
                  sm_scale: float, q_idx, w, idx_cache, q, kv_cache, new_idx=None, new_kv=None,
                  qb_candidates=(64, 256), u_max=None, path=None, outs=None, stream=None,
                  topk_order="position"):
    """Run a stack of DSA layers over one packed batch with IndexShare
    ("ref.py", build_index_share_map; "dsa_sparse_backend.py", __call__:
    a shared layer attends with the top-k of the nearest preceding full
    layer). Only library calls, in this order per layer i:

    1. the self-write of the batch's new tokens (dsa_paged_write_layer, one
       launch): new_kv[i] into kv_cache[i] and, on a full layer, its
       new_idx[slot] into idx_cache[slot] (skipped when new_kv is None);
    2. on a full layer: the indexer top-k (dsa_indexer_topk_ordered, in
       `topk_order`: "position" by default, since union and attention only
       see the set and gather faster in position order) into the layer's
       slot, then the block union sizes at each QB of qb_candidates
       (dsa_block_union without membership), which choose the attention
       (dsa_extend_attend_plan: a QB or the per-query path; this reads the
       union sizes on the host, a synchronisation of `stream`), and the
       full union tables at the chosen QB only;
    3. the attention of every layer with its source slot's selection:
       dsa_sparse_mla_extend at the chosen QB, or dsa_sparse_mla_decode
       (per query) on the packed batch.

    indexer_types lists "full" / "shared" per layer; q_idx, w, idx_cache
    (and new_idx) are lists indexed by slot (full layers in order); q,
    kv_cache, new_kv are lists indexed by layer. path forces "per_query" or
    a QB for every slot. Returns (outs, info): outs[i] bf16 [T, H, 512];
    info["topk"][slot], info["choice"][slot] (0 = per query, else the QB),
    info["counts"][slot] (QB -> blk_counts: every candidate when planned,
    else the forced QB only).
    """
    full_slot, src_slot, n_full = index_share_map(indexer_types)
    n_layers = len(indexer_types)
    torch = _torch()
    dev = q[0].device
    S, MP = _ragged(page_table, seq_lens, cu_q_lens, dev)
    T, H, _ = q[0].shape
    PS = kv_cache[0].shape[1]
    if len(q_idx) != n_full or len(w) != n_full or len(idx_cache) != n_full:
        raise ValueError(f"{n_full} full layers need {n_full} q_idx, w and idx_cache entries")
    if len(q) != n_layers or len(kv_cache) != n_layers:
        raise ValueError(f"{n_layers} layers need {n_layers} q and kv_cache entries")
    if new_kv is not None and (len(new_kv) != n_layers or new_idx is None
                               or len(new_idx) != n_full):
        raise ValueError("new_kv needs one entry per layer and new_idx one per full layer")
    qbs = [int(x) for x in qb_candidates]
    topk = [None] * n_full
    tables = [None] * n_full
    choice = [None] * n_full
    counts = [None] * n_full
    if outs is None:
        outs = [None] * n_layers
    for i in range(n_layers):
        slot = src_slot[i]
        own = full_slot.get(i)
        if new_kv is not None:
            paged_write_layer(new_idx[own] if own is not None else None,
                              idx_cache[own] if own is not None else None,
                              new_kv[i], kv_cache[i], page_table, seq_lens, cu_q_lens,
                              stream=stream)
        if own is not None:
            tk = indexer_topk(q_idx[own], w[own], idx_cache[own], page_table, seq_lens,
                              cu_q_lens, k, max_q_len, stream=stream, order=topk_order)
            topk[own] = tk
            ums = {qb: (u_max if u_max is not None else min(qb * k, S * MP)) for qb in qbs}
            tabs, cnts = {}, {}
            if path is None:
                # sizes only for the plan; membership only at the chosen QB
                for qb in qbs:
                    cnts[qb] = block_union(tk, seq_lens, cu_q_lens, PS, MP, qb, ums[qb],
                                           stream=stream, member=False)[1]
                um0 = min(ums.values()) if ums else (u_max or S * MP)
                choice[own] = extend_attend_plan(cnts, T, H, k, PS, um0)
            else:
                choice[own] = 0 if path == "per_query" else int(path)
                if choice[own] and choice[own] not in ums:
                    raise ValueError(f"forced QB {path} is not among qb_candidates")
            c = choice[own]
            if c:
                tabs[c] = (block_union(tk, seq_lens, cu_q_lens, PS, MP, c, ums[c],
                                       stream=stream), ums[c])
                cnts[c] = tabs[c][0][1]
            tables[own] = tabs
            counts[own] = cnts
        c = choice[slot]
        if c == 0:
            outs[i] = sparse_mla_decode(q[i], kv_cache[i], page_table, seq_lens, cu_q_lens,
                                        topk[slot], sm_scale, out=outs[i], stream=stream)
        else:
            (units, cnt, member), _um = tables[slot][c]
            outs[i] = sparse_mla_extend(q[i], kv_cache[i], page_table, seq_lens, cu_q_lens,
                                        units, cnt, member, c, sm_scale, out=outs[i],
                                        stream=stream)
    return outs, {"topk": topk, "choice": choice, "counts": counts,
                  "src_slot": src_slot, "full_slot": full_slot}
