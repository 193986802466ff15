"""Helpers for GPU parity tests: move seeded workloads to the device and
compare GPU results with the oracle."""
import sys

import numpy as np

import workloads as W

ATOL = 2e-2      # max-abs bound on attention outputs
RTOL_L2 = 5e-3   # relative L2 bound on attention outputs


def torch_mod():
    import torch

    return torch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16(a, dev):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def i32(a, dev):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def f32(a, dev):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)


class Dev:
    """Device copies of a workload's shared tensors (caches, table, lengths)."""

    def __init__(self, wl: W.Workload, dev="cuda", layers=None):
        self.wl = wl
        self.dev = dev
        self.page_table = i32(wl.page_table, dev)
        self.seq_lens = i32(wl.seq_lens, dev)
        self.idx_cache = wl.idx_cache.to_torch(dev)
        n = len(wl.kv_cache) if layers is None else layers
        self.kv_cache = [wl.kv_cache[i].to_torch(dev) for i in range(n)
                         if wl.kv_cache[i] is not None]

    def batch(self, name, layer=0):
        b = self.wl.batches[name]
        out = dict(cu=i32(b.cu_q_lens, self.dev), q_idx=bf16(b.q_idx, self.dev),
                   w=f32(b.w, self.dev))
        if b.q_mla and b.q_mla[layer] is not None:
            out["q"] = bf16(b.q_mla[layer], self.dev)
        return out


def to_np(t):
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return W.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def check_attention(got, ref, rows=None, what=""):
    """got, ref: float64 [T, H, Dv]; max-abs and relative-L2 bounds of bf16 attention."""
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    max_abs = float(err.max(initial=0.0))
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got))
    log(f"  {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    assert max_abs <= ATOL, f"{what}: max-abs {max_abs} > {ATOL}"
    assert rel <= RTOL_L2, f"{what}: rel-L2 {rel} > {RTOL_L2}"


def check_topk_rows_valid(topk, seq_lens, cu, k):
    """Properties every row must have at any size: -1 count, causality,
    distinct positions. Vectorised over rows."""
    T = topk.shape[0]
    seq = np.full(T, -1)
    pos = np.full(T, -1)
    for s in range(len(seq_lens)):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        seq[q0:q1] = s
        pos[q0:q1] = int(seq_lens[s]) - (q1 - q0) + np.arange(q1 - q0)
    inrow = seq >= 0
    n_valid = np.where(inrow, np.minimum(np.where(inrow, seq_lens[np.maximum(seq, 0)], 0),
                                         pos + 1), 0)
    n_valid = np.maximum(n_valid, 0)
    m = np.minimum(k, n_valid)
    cols = np.arange(k)[None, :]
    real = cols < m[:, None]
    assert ((topk >= 0) == real).all(), "wrong -1 padding count"
    assert (np.where(real, topk, -1) <= pos[:, None]).all(), "non-causal position"
    srt = np.sort(np.where(real, topk, -1), axis=1)
    dup = (srt[:, 1:] == srt[:, :-1]) & (srt[:, 1:] >= 0)
    assert not dup.any(), "duplicate position in a row"
