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
    "dsa_block_union_workspace": (_c_size, [_c_int] * 5),
    "dsa_block_union": (_c_int, [_vp, _vp, _vp] + [_c_int] * 7 + [_vp, _vp, _vp, _vp, _c_size,
                                                                  _vp]),
    "dsa_sparse_mla_decode_workspace": (_c_size, [_c_int] * 3),
    "dsa_sparse_mla_decode": (_c_int, [_vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp]
                              + [_c_int] * 6 + [_c_float, _vp, _vp, _c_size, _vp]),
    "dsa_sparse_mla_extend_workspace": (_c_size, [_c_int] * 4),
    "dsa_extend_attend_path": (_c_int, [_vp] + [_c_int] * 7),
    "dsa_index_share_map": (_c_int, [_vp, _c_int, _vp, _vp]),
    "dsa_indexer_page_topk_workspace": (_c_size, [_c_int] * 8),
    "dsa_indexer_page_topk": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _vp, _vp] + [_c_int] * 8
                              + [_vp, _vp, _c_size, _vp]),
    "dsa_page_tokens": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "dsa_paged_write": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _c_int, _c_int, _vp, _vp, _vp]
                        + [_c_int] * 4 + [_vp]),
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


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {nbytes} needed")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


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


def indexer_topk(q_idx, w, idx_cache, page_table, seq_lens, cu_q_lens, k: int,
                 max_q_len: int, out=None, workspace=None, stream=None):
    """Exact lightning-indexer top-k -> int32 [T, k] (dsa_indexer_topk)."""
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
        out = torch.empty((T, k), dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, 2, dev)
    nbytes = indexer_topk_workspace(T, S, H, D, PS, MP, k, max_q_len)
    ws = _workspace(nbytes, dev, workspace)
    st = load().dsa_indexer_topk(_ptr(q_idx), _ptr(w), _ptr(idx_cache), P, _ptr(page_table),
                                 _ptr(seq_lens), _ptr(cu_q_lens), T, S, H, D, PS, MP, k,
                                 max_q_len, _ptr(out), _ptr(ws), nbytes, _stream(stream))
    _check("dsa_indexer_topk", st)
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
        out = torch.empty((T, k_pages), dtype=torch.int32, device=dev)
    _need(out, "out", torch.int32, 2, dev)
    nbytes = indexer_page_topk_workspace(T, S, H, D, PS, MP, k_pages, max_q_len)
    ws = _workspace(nbytes, dev, workspace)
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
        out = torch.empty((T, kp * PS), dtype=torch.int32, device=dev)
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


def block_union_workspace(T, S, MP, QB, u_max) -> int:
    return load().dsa_block_union_workspace(T, S, MP, QB, u_max)


def block_union(topk, seq_lens, cu_q_lens, PS: int, MP: int, QB: int, u_max: int,
                out=None, workspace=None, stream=None):
    """Query-block union tables -> (units [nQB,u_max] i32, counts [nQB] i32,
    member [nQB,u_max,QB] u64) (dsa_block_union)."""
    torch = _torch()
    dev = topk.device
    _need(topk, "topk", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    _need(cu_q_lens, "cu_q_lens", torch.int32, 1, dev)
    T, k = topk.shape
    S = seq_lens.shape[0]
    nqb = (T + QB - 1) // QB
    if out is None:
        out = (torch.empty((nqb, u_max), dtype=torch.int32, device=dev),
               torch.empty((nqb,), dtype=torch.int32, device=dev),
               torch.empty((nqb, u_max, QB), dtype=torch.uint64, device=dev))
    units, counts, member = out
    nbytes = block_union_workspace(T, S, MP, QB, u_max)
    ws = _workspace(nbytes, dev, workspace)
    st = load().dsa_block_union(_ptr(topk), _ptr(seq_lens), _ptr(cu_q_lens), T, S, k, PS, MP, QB,
                                u_max, _ptr(units), _ptr(counts), _ptr(member), _ptr(ws), nbytes,
                                _stream(stream))
    _check("dsa_block_union", st)
    return units, counts, member


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
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    nbytes = sparse_mla_decode_workspace(T, H, k)
    ws = _workspace(nbytes, dev, workspace)
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
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
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
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    nbytes = sparse_mla_decode_workspace(T, H, kp * PS)
    ws = _workspace(nbytes, dev, workspace)
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
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    nbytes = sparse_mla_extend_workspace(T, H, QB, u_max)
    ws = _workspace(nbytes, dev, workspace)
    st = load().dsa_sparse_mla_extend(_ptr(q), _ptr(kv_cache), rs, P, _ptr(page_table),
                                      _ptr(seq_lens), _ptr(cu_q_lens), _ptr(units),
                                      _ptr(counts), _ptr(member), T, S, H, PS, MP, QB, u_max,
                                      float(sm_scale), _ptr(out), _ptr(ws) if ws is not None
                                      else None, nbytes, _stream(stream))
    _check("dsa_sparse_mla_extend", st)
    return out
