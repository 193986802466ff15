"""Seeded synthetic inputs for the DeepSeek-Sparse-Attention hot path.

This module only *makes data*: paged caches, page tables, ragged metadata,
query tensors and token selections, all from seeded NumPy generators. It
holds none of the method's arithmetic (no scoring, selection, union or
attention), so it can feed both the CPU oracle and the GPU library without
either of them depending on the other.

Value recipe (the pages print no data, so these follow the workload
descriptions of the decode and chunked-prefill configurations):

* indexer queries and keys: bf16 integers uniform in {-2..2};
* indexer head weights: fp32 uniform from {0.25, 0.5, 1, 2};
* MLA queries and latent rows: N(0, 1) rounded to bf16;
* physical page pool of ``S * MP`` pages, page table = a seeded permutation;
* every cache slot at a position >= kv_len, and every unused page, holds NaN
  in both caches, so any read outside the valid range shows up downstream.

bf16 tensors travel as ``uint16`` bit patterns (what the GPU reads);
``bf16_to_f64`` decodes them exactly for the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------
# bf16 encoding helpers (data conversion, not method arithmetic)
# ----------------------------------------------------------------------------
def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # round half to even on the dropped 16 bits; finite values cannot overflow
    # 32 bits here, NaN patterns are fixed below
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_to_f32(bits).astype(np.float64)


_INT_BF16 = f32_to_bf16(np.arange(-2, 3, dtype=np.float32))  # bits of -2..2
_W_CHOICES = np.array([0.25, 0.5, 1.0, 2.0], dtype=np.float32)


# ----------------------------------------------------------------------------
# Paged caches, stored compactly
# ----------------------------------------------------------------------------
class PagedCache:
    """A paged bf16 cache [num_pages, PS, D] kept as its live rows only.

    ``slots`` holds the ascending flat slot ids (page * PS + offset) of live
    tokens and ``rows`` their bf16 bits; every other slot is NaN. The full
    pool is materialised on demand: ``dense()`` on the host (small cases),
    ``to_torch()`` directly on the device, ``f64_view()`` as a read-only
    float64 view indexable like ``cache[pages, offsets]``.
    """

    def __init__(self, num_pages: int, PS: int, D: int, slots: np.ndarray, rows: np.ndarray):
        self.num_pages, self.PS, self.D = int(num_pages), int(PS), int(D)
        self.slots = np.asarray(slots, dtype=np.int64)
        self.rows = rows
        self.shape = (self.num_pages, self.PS, self.D)

    @property
    def nbytes(self) -> int:
        return self.num_pages * self.PS * self.D * 2

    def dense(self) -> np.ndarray:
        out = np.full((self.num_pages * self.PS, self.D), BF16_NAN, dtype=np.uint16)
        out[self.slots] = self.rows
        return out.reshape(self.shape)

    def __array__(self, dtype=None, copy=None):
        a = self.dense()
        return a if dtype is None else a.astype(dtype)

    def f64_view(self) -> "_F64Rows":
        return _F64Rows(self)

    def with_columns(self, extra: int) -> "PagedCache":
        """Same cache with ``extra`` NaN columns appended to every row."""
        pad = np.full((self.rows.shape[0], extra), BF16_NAN, dtype=np.uint16)
        return PagedCache(self.num_pages, self.PS, self.D + extra, self.slots,
                          np.concatenate([self.rows, pad], axis=1))

    def to_torch(self, device):
        import torch

        t = torch.full((self.num_pages * self.PS, self.D), float("nan"), dtype=torch.bfloat16,
                       device=device)
        rows = torch.from_numpy(np.ascontiguousarray(self.rows).view(np.int16)).view(torch.bfloat16)
        idx = torch.from_numpy(self.slots)
        t.index_copy_(0, idx.to(device), rows.to(device))
        return t.view(self.num_pages, self.PS, self.D)


class _F64Rows:
    """float64 view of a PagedCache: ``view[pages, offsets] -> [n, D]``."""

    def __init__(self, pc: PagedCache):
        self.pc = pc
        self.shape = pc.shape

    def __getitem__(self, idx):
        pages, offs = idx
        flat = np.asarray(pages, dtype=np.int64) * self.pc.PS + np.asarray(offs, dtype=np.int64)
        slots = self.pc.slots
        pos = np.minimum(np.searchsorted(slots, flat), max(slots.size - 1, 0))
        hit = slots[pos] == flat if slots.size else np.zeros(flat.shape, bool)
        out = bf16_to_f64(self.pc.rows[pos]) if slots.size else np.zeros(flat.shape + (self.pc.D,))
        out[~hit] = np.nan
        return out


# ----------------------------------------------------------------------------
# Workload container
# ----------------------------------------------------------------------------
@dataclass
class Batch:
    """One ragged batch of queries against the workload's caches."""

    cu_q_lens: np.ndarray  # int32 [S+1]
    q_idx: np.ndarray      # uint16 (bf16 bits) [T, H_idx, D_idx]
    w: np.ndarray          # float32 [T, H_idx]
    q_mla: List[np.ndarray]  # per layer: uint16 [T, H_mla, Dk]

    @property
    def T(self) -> int:
        return int(self.q_idx.shape[0])


@dataclass
class Workload:
    name: str
    S: int
    PS: int
    MP: int
    seq_lens: np.ndarray      # int32 [S]
    page_table: np.ndarray    # int32 [S, MP]
    idx_cache: PagedCache     # bf16 [P, PS, D_idx]
    kv_cache: List[PagedCache]  # per layer: bf16 [P, PS, Dk]
    H_idx: int
    D_idx: int
    k: int
    H_mla: int
    Dk: int
    Dv: int
    sm_scale: float
    batches: dict = field(default_factory=dict)  # name -> Batch
    QB: Sequence[int] = ()
    u_max: int = 0
    seed: int = 0

    @property
    def num_pages(self) -> int:
        return self.idx_cache.num_pages


# ----------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------
def _streams(seed: int, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(n)]


def _used_mask(seq_lens, page_table, num_pages, PS):
    """bool [num_pages, PS]: True where a slot holds a live token."""
    used = np.zeros((num_pages, PS), dtype=bool)
    S, MP = page_table.shape
    for s in range(S):
        n = int(seq_lens[s])
        full, rem = divmod(n, PS)
        if full:
            used[page_table[s, :full]] = True
        if rem:
            used[page_table[s, full], :rem] = True
    return used


def _int_cache(rng, used, D):
    P, PS = used.shape
    slots = np.flatnonzero(used.reshape(-1))
    vals = rng.integers(0, 5, size=(slots.size, D), dtype=np.int8)
    return PagedCache(P, PS, D, slots, _INT_BF16[vals])


_CHUNK_ROWS = 1 << 15  # rows drawn per call; fixed so the stream is reproducible


def _normal_cache(rng, used, D):
    P, PS = used.shape
    slots = np.flatnonzero(used.reshape(-1))
    rows = np.empty((slots.size, D), dtype=np.uint16)
    for i in range(0, slots.size, _CHUNK_ROWS):
        m = min(_CHUNK_ROWS, slots.size - i)
        rows[i : i + m] = f32_to_bf16(rng.standard_normal((m, D), dtype=np.float32))
    return PagedCache(P, PS, D, slots, rows)


def _int_tensor(rng, shape):
    return _INT_BF16[rng.integers(0, 5, size=shape, dtype=np.int8)]


def _normal_tensor(rng, shape):
    return f32_to_bf16(rng.standard_normal(shape, dtype=np.float32))


def _weights(rng, shape):
    return _W_CHOICES[rng.integers(0, 4, size=shape)]


def build(
    *,
    name: str,
    seed: int,
    S: int,
    kv_lens,
    PS: int,
    MP: int,
    batches: dict,
    H_idx: int,
    D_idx: int,
    k: int,
    H_mla: int = 16,
    Dk: int = 576,
    Dv: int = 512,
    sm_scale: Optional[float] = None,
    n_layers: int = 1,
    QB: Sequence[int] = (),
    u_max: int = 0,
    with_mla: bool = True,
    extra_pages: int = 0,
) -> Workload:
    """Generic seeded workload.

    ``kv_lens`` is a list of ints, or a callable ``rng -> int32[S]``.
    ``batches`` maps a batch name to its ``cu_q_lens`` list.
    The physical pool has ``S * MP + extra_pages`` pages; the page table is a
    seeded permutation of the first ``S * MP`` of them.
    Streams, in this fixed order: seq_lens, page_table, idx_cache, then per
    batch (q_idx, w, per-layer MLA q), then per-layer kv_cache.
    """
    n_batches = len(batches)
    rngs = _streams(seed, 3 + n_batches * (2 + n_layers) + n_layers)
    it = iter(rngs)
    r_len = next(it)
    if callable(kv_lens):
        seq_lens = np.asarray(kv_lens(r_len), dtype=np.int32)
    else:
        seq_lens = np.asarray(kv_lens, dtype=np.int32)
    assert seq_lens.shape == (S,)
    assert int(seq_lens.max(initial=0)) <= MP * PS, "kv_len exceeds page-table capacity"
    num_pages = S * MP + extra_pages
    page_table = next(it).permutation(S * MP).astype(np.int32).reshape(S, MP)
    used = _used_mask(seq_lens, page_table, num_pages, PS)
    idx_cache = _int_cache(next(it), used, D_idx)

    out_batches = {}
    for bname, cu in batches.items():
        cu = np.asarray(cu, dtype=np.int32)
        assert cu.shape == (S + 1,)
        T = int(cu[-1])
        q_idx = _int_tensor(next(it), (T, H_idx, D_idx))
        w = _weights(next(it), (T, H_idx))
        q_mla = []
        for _ in range(n_layers):
            r = next(it)
            q_mla.append(_normal_tensor(r, (T, H_mla, Dk)) if with_mla else None)
        out_batches[bname] = Batch(cu_q_lens=cu, q_idx=q_idx, w=w, q_mla=q_mla)

    kv_cache = []
    for _ in range(n_layers):
        r = next(it)
        kv_cache.append(_normal_cache(r, used, Dk) if with_mla else None)

    return Workload(
        name=name, S=S, PS=PS, MP=MP, seq_lens=seq_lens, page_table=page_table,
        idx_cache=idx_cache, kv_cache=kv_cache, H_idx=H_idx, D_idx=D_idx, k=k,
        H_mla=H_mla, Dk=Dk, Dv=Dv,
        sm_scale=float(sm_scale if sm_scale is not None else 1.0 / np.sqrt(192.0)),
        batches=out_batches, QB=tuple(QB), u_max=u_max, seed=seed,
    )


def decode_cu(S: int):
    return list(range(S + 1))


# ----------------------------------------------------------------------------
# The five named workloads
# ----------------------------------------------------------------------------
CONFIG_NAMES = {
    1: "tiny",
    2: "decode_batch_8x8192",
    3: "ragged_decode_64x4k-32k",
    4: "chunked_extend_4x13312_T4096",
    5: "long_extend_131072_T8192_indexshare4",
}


def config(cid: int, *, with_mla: bool = True, layers: Optional[int] = None) -> Workload:
    """Workload ``cid`` in 1..5, seeded with ``1000 + cid``."""
    seed = 1000 + cid
    if cid == 1:
        return build(
            name=CONFIG_NAMES[1], seed=seed, S=2, kv_lens=[100, 256], PS=16, MP=16,
            batches={"decode": [0, 1, 2], "extend": [0, 0, 32]},
            H_idx=4, D_idx=32, k=32, H_mla=4, n_layers=layers or 1,
            QB=(16, 64), u_max=32, with_mla=with_mla,
        )
    if cid == 2:
        return build(
            name=CONFIG_NAMES[2], seed=seed, S=8, kv_lens=[8192] * 8, PS=64, MP=128,
            batches={"decode": decode_cu(8)}, H_idx=32, D_idx=128, k=2048,
            H_mla=16, n_layers=layers or 1, with_mla=with_mla,
        )
    if cid == 3:
        return build(
            name=CONFIG_NAMES[3], seed=seed, S=64,
            kv_lens=lambda r: r.integers(4096, 32768, endpoint=True, size=64),
            PS=64, MP=512, batches={"decode": decode_cu(64)}, H_idx=32, D_idx=128,
            k=2048, H_mla=16, n_layers=layers or 1, with_mla=with_mla,
        )
    if cid == 4:
        return build(
            name=CONFIG_NAMES[4], seed=seed, S=4, kv_lens=[13312] * 4, PS=64, MP=208,
            batches={"extend": [0, 1024, 2048, 3072, 4096]}, H_idx=32, D_idx=128,
            k=2048, H_mla=16, n_layers=layers or 1, QB=(64, 256), u_max=832,
            with_mla=with_mla,
        )
    if cid == 5:
        return build(
            name=CONFIG_NAMES[5], seed=seed, S=1, kv_lens=[131072], PS=64, MP=2048,
            batches={"extend": [0, 8192]}, H_idx=32, D_idx=128, k=2048, H_mla=16,
            n_layers=layers or 4, QB=(256, 64), u_max=2048, with_mla=with_mla,
        )
    raise ValueError(f"unknown config {cid}")


# ----------------------------------------------------------------------------
# Seeded token selections with locality (attend-stage inputs)
# ----------------------------------------------------------------------------
def locality_selection(seq_lens, cu_q_lens, k: int, seed: int, *, sinks: int = 64,
                       window: int = 1024, T: Optional[int] = None) -> np.ndarray:
    """int32 [T, k] seq-local positions, one row per packed query.

    For a query at absolute position p (p = kv_len - q_len + offset in chunk):
    the first ``sinks`` positions, the last ``window`` causal positions
    (p - window + 1 .. p) and positions drawn uniformly without replacement
    from the rest of 0..p, until exactly min(k, p + 1) positions are chosen.
    Each row is sorted ascending and padded with -1. Rows outside every
    sequence are all -1.
    """
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    if T is None:
        T = int(cu[-1])
    out = np.full((T, k), -1, dtype=np.int32)
    for s in range(len(seq_lens)):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        n = q1 - q0
        for i in range(n):
            t = q0 + i
            if t >= T:
                break
            p = int(seq_lens[s]) - n + i
            if p < 0:
                continue
            if p + 1 <= k:
                out[t, : p + 1] = np.arange(p + 1)
                continue
            lo_win = max(0, p - window + 1)
            base = np.union1d(np.arange(min(sinks, p + 1)), np.arange(lo_win, p + 1))
            need = k - base.size
            if need > 0:
                # remaining causal positions are the gap [sinks, lo_win)
                gap_lo = min(sinks, p + 1)
                gap = lo_win - gap_lo
                pick = rng.choice(gap, size=need, replace=False) + gap_lo
                sel = np.union1d(base, pick)
            else:
                sel = base[:k]
            out[t, : sel.size] = sel
    return out


def random_selection(seq_lens, cu_q_lens, k: int, seed: int, *, fill: float = 0.7,
                     T: Optional[int] = None, allow_out_of_range: bool = False) -> np.ndarray:
    """int32 [T, k] duplicate-free random seq-local positions per query.

    Each row holds min(k, round(fill * n)) causal positions (n = p + 1) in
    random order, the rest -1 interleaved at random slots. With
    ``allow_out_of_range`` a few entries are replaced by positions in
    [p + 1, kv_len) (non-causal) so masks can be exercised.
    """
    rng = np.random.default_rng(np.random.SeedSequence(seed))
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    if T is None:
        T = int(cu[-1])
    out = np.full((T, k), -1, dtype=np.int32)
    for s in range(len(seq_lens)):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        n_q = q1 - q0
        kv = int(seq_lens[s])
        for i in range(n_q):
            t = q0 + i
            if t >= T:
                break
            p = kv - n_q + i
            if p < 0:
                continue
            m = min(k, max(1, int(round(fill * (p + 1)))))
            sel = rng.choice(p + 1, size=m, replace=False).astype(np.int32)
            if allow_out_of_range and p + 1 < kv and m >= 2:
                extra = rng.integers(p + 1, kv, size=max(1, m // 8))
                sel = np.unique(np.concatenate([sel[: m - extra.size], extra])).astype(np.int32)
                rng.shuffle(sel)
            slots = rng.choice(k, size=sel.size, replace=False)
            out[t, slots] = sel
    return out
