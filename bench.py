#!/usr/bin/env python3
"""Benchmark of the DeepSeek-Sparse-Attention hot path on one MI355X.

Headline (the JSON line's `value`): extend ms per layer on the long-context
IndexShare workload (one request, 131072-token context, its final
8192-token chunk, page size 64; indexer 32 heads x 128, k = 2048; four
layers of sparse MLA with 16 heads, the first full, three sharing its
top-k). One step is the four layers in order, each timed end to end:

  full layer    the self-write of the chunk's indexer keys and latent rows
                (one launch), the indexer top-k, the query-block union of
                the attend's selection (its block sizes only, which the
                plan reads, when the attention runs per query), and the
                sparse MLA attention;
  shared layer  the self-write of its latent rows and the attention with the
                full layer's selection and union.

The attention runs on the path the library's plan picks from the union
sizes (per query, or query blocks of 64 / 256). As the workload prescribes
for timing, union and attention take the seeded locality selection (first 64
positions, last 1024, uniform rest); the same step with the indexer's own
selection is reported beside it. value = step ms / 4 layers.

Beside it, in the same line: the decode batch (8 x 8192) and the ragged
decode (64 x [4K, 32K]) in tokens/s, the chunked extend (4 x (12288 + 1024))
at QB 64 and 256 and per query, per-kernel durations warm and with cold
caches (median, p10, p90), the copy-kernel bandwidth, and the CPU oracle's
per-stage time on the host cores.

Inputs are seeded synthetic tensors already resident in HBM when a timed
region starts. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--no-cpu-baseline]
                  [--only all|long|decode|ragged|extend|copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode tok/s & extend ms/layer (indexer top-k + sparse MLA), % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
DK, DV = 576, 512
FLUSH_BYTES = 1 << 30           # four times the 256 MB infinity cache


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10,
                   help="timed steps of the headline (long-context) step")
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--only", choices=["all", "long", "decode", "ragged", "extend", "copy"],
                   default="all",
                   help="run one workload alone (for per-workload profiles); 'copy' times a "
                        "plain device copy, the scale of the HBM byte counters")
    p.add_argument("--cold-reps", type=int, default=0,
                   help="repetitions of the cold/warm per-kernel statistics (0: per workload "
                        "default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time of the oracle baseline sample")
    return p.parse_args(argv)


# ----------------------------------------------------------------------------
# device inputs
# ----------------------------------------------------------------------------
def _i32(a):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _bf16(a):
    import numpy as np
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _dev_inputs(wl, bname, layers=1):
    import numpy as np
    import torch

    b = wl.batches[bname]
    return dict(
        page_table=_i32(wl.page_table), seq_lens=_i32(wl.seq_lens), cu=_i32(b.cu_q_lens),
        idx_cache=wl.idx_cache.to_torch("cuda"),
        kv_cache=[wl.kv_cache[i].to_torch("cuda") for i in range(layers)],
        q_idx=_bf16(b.q_idx), w=torch.from_numpy(b.w).cuda(),
        q=[_bf16(b.q_mla[i]) for i in range(layers)],
        max_q_len=int(np.diff(b.cu_q_lens).max()),
    )


def _rows_seq(wl, cu):
    import numpy as np

    T = int(cu[-1])
    seq = np.full(T, -1, dtype=np.int64)
    pos = np.full(T, -1, dtype=np.int64)
    for s in range(wl.S):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        seq[q0:q1] = s
        pos[q0:q1] = int(wl.seq_lens[s]) - (q1 - q0) + np.arange(q1 - q0)
    return seq, pos


def _chunk_rows(cache, wl, cu):
    """bf16 device tensor [T, D]: the workload cache's row at each packed
    row's own position, i.e. the new tokens the layer's self-write puts into
    the cache (writing them back leaves the workload unchanged)."""
    import numpy as np

    seq, pos = _rows_seq(wl, cu)
    flat = wl.page_table[seq, pos // wl.PS].astype(np.int64) * wl.PS + pos % wl.PS
    idx = np.searchsorted(cache.slots, flat)
    assert (cache.slots[idx] == flat).all()
    return _bf16(cache.rows[idx])


def _row_valid_counts(wl, cu):
    """n_valid per packed row (positions j < kv and j <= abs_q)."""
    import numpy as np

    seq, pos = _rows_seq(wl, cu)
    kv = np.where(seq >= 0, wl.seq_lens[np.maximum(seq, 0)], 0)
    return np.clip(np.minimum(pos + 1, kv), 0, None)


# ----------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------
def _timed(step, steps, warmup):
    """ms per step over exactly `steps` calls after `warmup` untimed ones,
    bracketed by device synchronisation; events on the current stream (the
    stream every library call here is launched on)."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _graph_timed(step, steps, warmup):
    """ms per replay of one step captured as a HIP graph (torch.cuda.CUDAGraph):
    the step's launches are replayed as one submission. The step runs eagerly
    first, so that one-time state (kernel attributes, static scratch) is set
    outside the capture; every buffer it uses is preallocated."""
    import torch

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def _kernel_times(dsa, step, steps):
    """{kernel: (launches per step, average ms per launch)} over `steps`
    steps, from the library's per-launch HIP events (recorded on the launch
    stream of each kernel)."""
    import torch

    torch.cuda.synchronize()
    dsa.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = dsa.profile_read()
    dsa.profile_enable(False)
    return {k: (n // steps, tot / n) for k, (n, tot) in prof.items()}


def _kernel_stats(dsa, step, reps, cold):
    """Per-kernel launch duration statistics over `reps` steps, one step per
    record: {kernel: [average ms per launch in each rep]}. With `cold`, a
    1 GiB buffer (four times the 256 MB infinity cache) is read before every
    step, outside the library's timed launches: a read leaves clean lines,
    so the next kernel pays no write-back of the flush."""
    import torch

    flush = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if cold else None
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    per = {}
    step()
    for _ in range(reps):
        if cold:
            torch.sum(flush, dim=0, out=sink)
        torch.cuda.synchronize()
        dsa.profile_enable(True)
        step()
        torch.cuda.synchronize()
        prof = dsa.profile_read()
        dsa.profile_enable(False)
        for k, (n, tot) in prof.items():
            per.setdefault(k, []).append(tot / n)
    del flush
    return per


def _pct(xs):
    import numpy as np

    a = np.asarray(xs, dtype=np.float64) * 1e3
    return {"median_us": round(float(np.median(a)), 2),
            "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "reps": int(a.size)}


def _roofline_entry(bound, work, ms):
    """work = algorithmic bytes (hbm) or flops (mfma) of ONE launch."""
    if bound == "hbm":
        achieved = work / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = work / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}


def _kernel_table(kt, warm, cold, work):
    """One entry per kernel: the timed pass's average launch, warm and cold
    statistics, and for kernels with algorithmic work its roofline fraction
    (cold median first: the primary HBM measure; then warm and average)."""
    out = {}
    for name, (n, avg) in kt.items():
        e = {"launches_per_step": n, "avg_us": round(avg * 1e3, 2)}
        if name in warm:
            e["warm"] = _pct(warm[name])
        if name in cold:
            e["cold"] = _pct(cold[name])
        if name in work:
            bound, w = work[name]
            e["bound"], e["work_per_launch"] = bound, int(w)
            if name in cold:
                e["frac_cold_median"] = _roofline_entry(bound, w, e["cold"]["median_us"] / 1e3)["frac"]
            if name in warm:
                e["frac_warm_median"] = _roofline_entry(bound, w, e["warm"]["median_us"] / 1e3)["frac"]
            e["frac_avg"] = _roofline_entry(bound, w, avg)["frac"]
        out[name] = e
    return out


INDEXER_KERNELS = ("idx_score_stream", "idx_score_flat", "idx_score_regs", "idx_score_tiles",
                   "topk_select", "idx_score_topk", "topk_order", "topk_merge",
                   "topk_rows_ascending", "topk_rows_bitmap")

# Sources whose text decides each kernel's machine code.
KERNEL_SOURCES = {
    "idx_score_stream": "indexer.hip", "idx_score_flat": "indexer.hip",
    "idx_score_regs": "indexer.hip", "idx_score_tiles": "indexer.hip", "topk_select": "indexer.hip",
    "idx_score_topk": "indexer.hip", "topk_order": "indexer.hip", "topk_merge": "indexer.hip",
    "topk_rows_ascending": "indexer.hip", "topk_rows_bitmap": "indexer.hip",
    "mla_decode_partial": "mla.hip", "mla_decode_combine": "mla.hip",
    "mla_decode_combine_wide": "mla.hip", "mla_extend_qblock": "mla.hip",
    "union_clear": "union.hip", "union_mark": "union.hip", "union_compact": "union.hip",
    "union_member": "union.hip", "page_pool": "indexer.hip", "page_token_list": "indexer.hip",
    "paged_write_rows": "cache_write.hip",
}


def kernel_source_hash(kernel):
    """sha256 over the kernel's source file and the shared device header."""
    import hashlib

    csrc = os.path.join(ROOT, "sparse_attention_relu_amd", "csrc")
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES.get(kernel, "indexer.hip"), "common.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary
    profiles/traffic_<kernel>_<workload>.txt, or None when there is none or
    the kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != kernel_source_hash(kernel):
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _dominant(kt):
    return max(kt, key=lambda nm: kt[nm][0] * kt[nm][1])


def _headline_roofline(kt, kernels, work, workload):
    dom = _dominant({k: v for k, v in kt.items() if k in work})
    bound, w = work[dom]
    n, avg = kt[dom]
    roof = _roofline_entry(bound, w, avg)
    roof.update({"traffic": measured_traffic(dom, workload), "kernel": dom,
                 "work_per_launch": int(w), "avg_launch_us": round(avg * 1e3, 2),
                 "launches_per_step": n, "measured_over": "the timed steps (library events)"})
    e = kernels.get(dom, {})
    if "cold" in e:
        roof["cold"] = dict(e["cold"], frac=e.get("frac_cold_median"))
    if "warm" in e:
        roof["warm"] = dict(e["warm"], frac=e.get("frac_warm_median"))
    return roof


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def bench_decode(dsa, wl, steps, warmup, reps):
    """One DSA decode layer: indexer top-k, then sparse MLA decode."""
    import numpy as np
    import torch

    d = _dev_inputs(wl, "decode")
    b = wl.batches["decode"]
    T, k, H = b.T, wl.k, wl.H_mla
    topk = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda")
    ws_i = torch.empty(max(1, dsa.indexer_topk_workspace(T, wl.S, wl.H_idx, wl.D_idx, wl.PS,
                                                         wl.MP, k, 1)), dtype=torch.uint8,
                       device="cuda")
    ws_d = torch.empty(max(1, dsa.sparse_mla_decode_workspace(T, H, k)), dtype=torch.uint8,
                       device="cuda")

    def step():
        dsa.indexer_topk(d["q_idx"], d["w"], d["idx_cache"], d["page_table"], d["seq_lens"],
                         d["cu"], k, 1, out=topk, workspace=ws_i)
        dsa.sparse_mla_decode(d["q"][0], d["kv_cache"][0], d["page_table"], d["seq_lens"],
                              d["cu"], topk, wl.sm_scale, out=out, workspace=ws_d)

    ms = _timed(step, steps, warmup)
    kt = _kernel_times(dsa, step, steps)
    warm = _kernel_stats(dsa, step, reps, cold=False)
    cold = _kernel_stats(dsa, step, reps, cold=True)
    ms_graph = _graph_timed(step, steps, warmup)

    nval = _row_valid_counts(wl, b.cu_q_lens)
    n_sel = int((topk >= 0).sum())
    D, Hi, PS = wl.D_idx, wl.H_idx, wl.PS
    score_bytes = (int(nval.sum()) * (D * 2 + 4) + T * Hi * (D * 2 + 4)
                   + int(np.ceil(nval / PS).sum()) * 4)
    work = {
        "idx_score_stream": ("hbm", score_bytes),
        "idx_score_flat": ("hbm", score_bytes),
        "idx_score_regs": ("hbm", score_bytes),
        "topk_select": ("hbm", int(nval.sum()) * 4 + T * k * 4),
        "mla_decode_partial": ("hbm", n_sel * DK * 2 + T * k * 4 + T * H * DK * 2),
    }
    kernels = _kernel_table(kt, warm, cold, work)

    def part(names):
        return sum(kt[nm][0] * kt[nm][1] for nm in names if nm in kt)

    cold_step = [sum(v[i] * kt[k_][0] for k_, v in cold.items() if k_ in kt)
                 for i in range(reps)]
    return {"workload": wl.name, "seqs": wl.S, "tokens": int(wl.seq_lens.sum()),
            "tok_s": round(T / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
            "graph": {"ms_per_step": round(ms_graph, 5), "tok_s": round(T / (ms_graph * 1e-3), 1),
                      "note": "the same step captured once as a HIP graph and replayed"},
            "indexer_ms": round(part(INDEXER_KERNELS), 5),
            "attend_ms": round(part(("mla_decode_partial", "mla_decode_combine",
                                     "mla_decode_combine_wide")), 5),
            "cold_kernel_sum_ms_median": round(float(np.median(cold_step)), 5),
            "roofline": _headline_roofline(kt, kernels, work, wl.name),
            "kernels": kernels, "page_decode": bench_page_decode(dsa, wl, d, steps, warmup)}


def bench_page_decode(dsa, wl, d, steps, warmup):
    """The same decode layer with page-level selection: the page top-k
    (k_pages = k / PS pages, max-pooled page scores), then sparse MLA over
    every valid position of those pages (page lists read directly)."""
    import torch

    b = wl.batches["decode"]
    T, H, PS = b.T, wl.H_mla, wl.PS
    kp = max(1, wl.k // PS)
    pages = torch.empty((T, kp), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda")
    ws_i = torch.empty(max(1, dsa.indexer_page_topk_workspace(T, wl.S, wl.H_idx, wl.D_idx, PS,
                                                              wl.MP, kp, 1)),
                       dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(max(1, dsa.sparse_mla_decode_workspace(T, H, kp * PS)),
                       dtype=torch.uint8, device="cuda")

    def step():
        dsa.indexer_page_topk(d["q_idx"], d["w"], d["idx_cache"], d["page_table"],
                              d["seq_lens"], d["cu"], kp, 1, out=pages, workspace=ws_i)
        dsa.sparse_mla_decode_pages(d["q"][0], d["kv_cache"][0], d["page_table"],
                                    d["seq_lens"], d["cu"], pages, wl.sm_scale, out=out,
                                    workspace=ws_d)

    ms = _timed(step, steps, warmup)
    kt = _kernel_times(dsa, step, steps)
    return {"k_pages": kp, "ms_per_step": round(ms, 5), "tok_s": round(T / (ms * 1e-3), 1),
            "kernels_us": {nm: round(avg * 1e3, 2) for nm, (n, avg) in kt.items()}}


# ----------------------------------------------------------------------------
# extend
# ----------------------------------------------------------------------------
class ExtendLayers:
    """Device state of an extend workload: caches, queries, the chunk's new
    rows, the indexer's and the locality selection, union tables per QB."""

    def __init__(self, dsa, wl):
        import numpy as np
        import torch

        import workloads as W

        self.dsa, self.wl = dsa, wl
        self.layers = len(wl.kv_cache)
        b = wl.batches["extend"]
        self.b = b
        self.d = _dev_inputs(wl, "extend", layers=self.layers)
        self.T, self.k, self.H = b.T, wl.k, wl.H_mla
        cu = b.cu_q_lens
        self.new_idx = _chunk_rows(wl.idx_cache, wl, cu)
        self.new_kv = [_chunk_rows(wl.kv_cache[i], wl, cu) for i in range(self.layers)]
        self.loc = _i32(W.locality_selection(wl.seq_lens, cu, wl.k, 100 + int(wl.seed) - 1000))
        self.topk = torch.empty((self.T, self.k), dtype=torch.int32, device="cuda")
        self.ws_i = torch.empty(dsa.indexer_topk_workspace(self.T, wl.S, wl.H_idx, wl.D_idx,
                                                           wl.PS, wl.MP, self.k,
                                                           self.d["max_q_len"]),
                                dtype=torch.uint8, device="cuda")
        self.ws_d = torch.empty(max(1, dsa.sparse_mla_decode_workspace(self.T, self.H, self.k)),
                                dtype=torch.uint8, device="cuda")
        self.outs = [torch.empty((self.T, self.H, DV), dtype=torch.bfloat16, device="cuda")
                     for _ in range(self.layers)]
        self.tables = {}
        self.u_max = wl.u_max
        for QB in (64, 256):
            nqb = (self.T + QB - 1) // QB
            self.tables[QB] = dict(
                units=torch.empty((nqb, self.u_max), dtype=torch.int32, device="cuda"),
                counts=torch.empty((nqb,), dtype=torch.int32, device="cuda"),
                member=torch.empty((nqb, self.u_max, QB), dtype=torch.uint64, device="cuda"),
                ws=torch.empty(max(1, dsa.block_union_workspace(self.T, wl.S, wl.MP, QB,
                                                                self.u_max)),
                               dtype=torch.uint8, device="cuda"))
        self.nval = _row_valid_counts(wl, cu)
        self.seq, _ = _rows_seq(wl, cu)
        self.np = np

    # one library call each ------------------------------------------------
    def write(self, i, full):
        d = self.d
        self.dsa.paged_write_layer(self.new_idx if full else None,
                                   d["idx_cache"] if full else None, self.new_kv[i],
                                   d["kv_cache"][i], d["page_table"], d["seq_lens"], d["cu"])

    def indexer(self):
        # position order, as the library's layer loop asks for its attention feed
        d = self.d
        self.dsa.indexer_topk(d["q_idx"], d["w"], d["idx_cache"], d["page_table"],
                              d["seq_lens"], d["cu"], self.k, d["max_q_len"], out=self.topk,
                              workspace=self.ws_i, order="position")

    def union(self, sel, QB, member=True):
        t = self.tables[QB]
        d = self.d
        self.dsa.block_union(sel, d["seq_lens"], d["cu"], self.wl.PS, self.wl.MP, QB,
                             self.u_max, out=(t["units"], t["counts"], t["member"]),
                             workspace=t["ws"], member=member)

    def attend(self, i, sel, path):
        d = self.d
        if path == 0:
            self.dsa.sparse_mla_decode(d["q"][i], d["kv_cache"][i], d["page_table"],
                                       d["seq_lens"], d["cu"], sel, self.wl.sm_scale,
                                       out=self.outs[i], workspace=self.ws_d)
        else:
            t = self.tables[path]
            self.dsa.sparse_mla_extend(d["q"][i], d["kv_cache"][i], d["page_table"],
                                       d["seq_lens"], d["cu"], t["units"], t["counts"],
                                       t["member"], path, self.wl.sm_scale, out=self.outs[i])

    # ----------------------------------------------------------------------
    def plan(self, sel):
        """The library's choice (0 = per query, else QB) for a selection,
        from its unions at QB 64 and 256 (read on the host, before timing)."""
        import torch

        for QB in (64, 256):
            self.union(sel, QB)
        torch.cuda.synchronize()
        counts = {QB: self.tables[QB]["counts"].cpu().numpy() for QB in (256, 64)}
        choice = self.dsa.extend_attend_plan(counts, self.T, self.H, self.k, self.wl.PS,
                                             self.u_max)
        return choice, counts

    def step_fn(self, sel_kind, path, layers=None, full_first=True):
        """One pass over `layers` layers (all by default): write, then on the
        full layer indexer top-k and the union (the block sizes a plan reads,
        at QB 256, when the attention runs per query; the full tables at the
        attention's QB otherwise), then the attention; `sel_kind` "locality"
        or "indexer" feeds union and attention."""
        n = self.layers if layers is None else layers
        sel = self.loc if sel_kind == "locality" else self.topk
        union_qb = path if path else 256

        def step():
            for i in range(n):
                full = full_first and i == 0
                self.write(i, full)
                if full:
                    self.indexer()
                    self.union(sel, union_qb, member=bool(path))
                self.attend(i, sel, path)
        return step

    def work(self, sel_np, QB_counts):
        """Algorithmic bytes or flops per launch of each kernel."""
        np = self.np
        wl = self.wl
        T, k, H = self.T, self.k, self.H
        n_sel = int((sel_np >= 0).sum())
        idx_flops = 2 * wl.H_idx * wl.D_idx * int(self.nval.sum())
        w = {"idx_score_tiles": ("mfma", idx_flops),
             "idx_score_topk": ("mfma", idx_flops),
             "topk_select": ("hbm", int(self.nval.sum()) * 4 + T * k * 4),
             "topk_order": ("hbm", T * k * (8 + 4)),
             "topk_rows_ascending": ("hbm", T * k * (4 + 4)),
             "topk_rows_bitmap": ("hbm", T * k * (4 + 4)),
             "mla_decode_partial": ("hbm", n_sel * DK * 2 + T * k * 4 + T * H * DK * 2),
             "paged_write_rows": ("hbm", T * (wl.D_idx + DK) * 2 * 2)}
        for QB, cnt in QB_counts.items():
            w[f"mla_extend_qblock@{QB}"] = ("mfma", int(np.minimum(cnt, self.u_max).sum())
                                            * QB * H * wl.PS * (DK + DV) * 2)
        return w, n_sel

    def redundancy(self, sel_np, counts):
        np = self.np
        keys = np.where(sel_np >= 0, self.seq[:, None] * self.wl.MP + sel_np // self.wl.PS, -1)
        per_query = sum(len(np.unique(r[r >= 0])) for r in keys)
        distinct = len(np.unique(keys[keys >= 0]))
        out = {"pages_distinct": distinct,
               "per_query": round(per_query / max(distinct, 1), 1)}
        for QB, c in counts.items():
            out[f"qblock_{QB}"] = round(float(c.sum()) / max(distinct, 1), 2)
        return out


def _attend_only(E, i, sel, path, steps):
    """ms per launch sequence of one layer's attention alone, and its
    per-kernel durations."""
    f = lambda: E.attend(i, sel, path)  # noqa: E731
    ms = _timed(f, steps, 1)
    return ms, _kernel_times(E.dsa, f, steps)


def bench_extend_workload(dsa, wl, steps, warmup, reps):
    """Extend layers of a workload: the planned path, every path timed on
    one layer, the end-to-end step (all layers), full and shared layers."""
    import numpy as np

    E = ExtendLayers(dsa, wl)
    res = {"workload": wl.name, "layers": E.layers, "T": E.T, "k": E.k,
           "step": "per layer: self-write; full layer: indexer top-k + union (sizes only "
                   "when per query); attention"}
    # the indexer once (its selection is the secondary feed)
    E.indexer()
    sel_np = {"locality": E.loc.cpu().numpy(), "indexer": E.topk.cpu().numpy()}
    choice, counts = {}, {}
    for kind in ("locality", "indexer"):
        choice[kind], counts[kind] = E.plan(E.loc if kind == "locality" else E.topk)
    res["attend_path_chosen"] = {kd: ("per_query" if c == 0 else f"qblock{c}")
                                 for kd, c in choice.items()}
    res["union_per_block"] = {f"{kd}_qb{QB}": {"min": int(c.min()),
                                              "mean": round(float(c.mean()), 1),
                                              "max": int(c.max())}
                              for kd in counts for QB, c in counts[kd].items()}
    res["redundant_fetch"] = {kd: E.redundancy(sel_np[kd], counts[kd]) for kd in counts}

    # end-to-end steps (all layers), locality selection first (the timed feed)
    steps_out = {}
    kt_main = None
    for kind in ("locality", "indexer"):
        path = choice[kind]
        E.union(E.loc if kind == "locality" else E.topk, path if path else 256)
        f = E.step_fn(kind, path)
        ms = _timed(f, steps, warmup)
        kt = _kernel_times(dsa, f, steps)
        steps_out[kind] = {"ms_per_step": round(ms, 4), "ms_per_layer": round(ms / E.layers, 4),
                           "path": res["attend_path_chosen"][kind]}
        if kind == "locality":
            kt_main = kt
            if E.layers > 1:
                ms_full = _timed(E.step_fn(kind, path, layers=1), steps, 1)
                ms_shared = _timed(E.step_fn(kind, path, layers=1, full_first=False), steps, 1)
                steps_out[kind].update({"ms_full_layer": round(ms_full, 4),
                                        "ms_shared_layer": round(ms_shared, 4)})
    res["steps"] = steps_out
    path = choice["locality"]
    f_main = E.step_fn("locality", path)
    E.union(E.loc, path if path else 256)
    warm = _kernel_stats(dsa, f_main, reps, cold=False)
    cold = _kernel_stats(dsa, f_main, reps, cold=True)

    # every attention path on one layer, locality selection
    w, n_sel = E.work(sel_np["locality"], counts["locality"])
    paths = {}
    for p in (0, 64, 256):
        E.union(E.loc, p if p else 256)
        ms, kt = _attend_only(E, 0, E.loc, p, max(2, steps // 2))
        name = "per_query" if p == 0 else f"qblock{p}"
        e = {"ms": round(ms, 4), "kernels_us": {nm: round(a * 1e3, 2) for nm, (n, a) in kt.items()}}
        if p == 0:
            e["roofline"] = _roofline_entry("hbm", w["mla_decode_partial"][1],
                                            kt["mla_decode_partial"][1])
            e["gathered_bytes"] = int(w["mla_decode_partial"][1])
        else:
            ex = w[f"mla_extend_qblock@{p}"][1]
            useful = n_sel * E.H * (DK + DV) * 2
            e["roofline_executed"] = _roofline_entry("mfma", ex, kt["mla_extend_qblock"][1])
            e["roofline_useful"] = _roofline_entry("mfma", useful, kt["mla_extend_qblock"][1])
            e["executed_tflop"] = round(ex / 1e12, 3)
            e["useful_tflop"] = round(useful / 1e12, 3)
        paths[name] = e
    res["attend_paths_one_layer"] = paths

    work = {k_: v for k_, v in w.items() if "@" not in k_}
    if path:
        work["mla_extend_qblock"] = w[f"mla_extend_qblock@{path}"]
    res["kernels"] = _kernel_table(kt_main, warm, cold, work)
    res["roofline"] = _headline_roofline(kt_main, res["kernels"], work, wl.name)
    res["indexer_ms"] = round(sum(kt_main[nm][1] for nm in INDEXER_KERNELS if nm in kt_main), 4)
    return res


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores, per stage
# ----------------------------------------------------------------------------
def cpu_baseline(wl, seconds):
    """The oracle's stages on a bounded sample of the long-context layer,
    scaled to ms per layer (same unit as the headline): score and top-k per
    row (the indexer's own rows), the union of one query block and the
    attention per row (the locality selection, as the timed step), each
    extrapolated to the workload's rows, blocks and four layers."""
    import numpy as np
    import oracle
    import workloads as W
    from threadpoolctl import threadpool_info
    from workloads import bf16_to_f64

    b = wl.batches["extend"]
    cu = b.cu_q_lens
    T = b.T
    QB = 256
    seq, pos = oracle.query_rows(wl.seq_lens, cu, T)
    q_idx, w = bf16_to_f64(b.q_idx), b.w.astype(np.float64)
    icache = wl.idx_cache.f64_view()
    budget = seconds / 3.0
    rng = np.random.default_rng(5)
    # score, then top-k, row by row (the oracle's own stage functions)
    t_score = t_topk = 0.0
    n_rows = 0
    t_end = time.perf_counter() + budget
    while time.perf_counter() < t_end or n_rows == 0:
        t = int(rng.integers(T))
        s = int(seq[t])
        n = oracle.n_valid_keys(wl.seq_lens[s], pos[t])
        t0 = time.perf_counter()
        keys = np.asarray(oracle.gather_rows(icache, wl.page_table, s, np.arange(n)))
        sc = oracle.indexer_scores(q_idx[t], w[t], keys)
        t1 = time.perf_counter()
        oracle.canonical_order(sc)[: min(wl.k, n)]
        t2 = time.perf_counter()
        t_score += t1 - t0
        t_topk += t2 - t1
        n_rows += 1
    loc = W.locality_selection(wl.seq_lens, cu, wl.k, 100 + int(wl.seed) - 1000)
    t0 = time.perf_counter()
    oracle.block_union(loc, wl.seq_lens, cu, wl.PS, wl.MP, QB, wl.u_max, blocks=[0])
    t_union = time.perf_counter() - t0
    q = bf16_to_f64(b.q_mla[0])
    kv = wl.kv_cache[0].f64_view()
    t_att, n_att = 0.0, 0
    t_end = time.perf_counter() + budget
    while time.perf_counter() < t_end or n_att == 0:
        t = int(rng.integers(T))
        t0 = time.perf_counter()
        oracle.sparse_mla(q, kv, wl.page_table, wl.seq_lens, cu, loc, wl.sm_scale, wl.Dv,
                          rows=[t])
        t_att += time.perf_counter() - t0
        n_att += 1
    layers = len(wl.kv_cache)
    nqb = (T + QB - 1) // QB
    stage_ms = {"score": t_score / n_rows * T * 1e3, "topk": t_topk / n_rows * T * 1e3,
                "union": t_union * nqb * 1e3, "attend_per_layer": t_att / n_att * T * 1e3}
    per_layer = (stage_ms["score"] + stage_ms["topk"] + stage_ms["union"]
                 + layers * stage_ms["attend_per_layer"]) / layers
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": round(per_layer, 1), "unit": "ms/layer", "cores": max(threads, 1),
            "kind": "oracle",
            "stages_ms_full_workload": {k_: round(v, 1) for k_, v in stage_ms.items()},
            "sample": f"{wl.name}: score and top-k of {n_rows} random rows, the union of one "
                      f"{QB}-row block, the attention of {n_att} random rows (locality "
                      f"selection), fp64 NumPy, each stage scaled to the workload's {T} rows, "
                      f"{nqb} blocks and {layers} layers"}


# ----------------------------------------------------------------------------
def copy_bandwidth(mib=1024, reps=10, verbose=False):
    """A plain device copy of known size (the runtime's copy kernel): its
    bandwidth, and under a counter profiler the byte scale of FETCH_SIZE /
    WRITE_SIZE per dispatch."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    r = {"bytes_read": n * 4, "bytes_written": n * 4, "ms": round(ms, 4),
         "GB_s": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}
    r["frac_of_peak"] = round(r["GB_s"] / HBM_PEAK_GBS, 4)
    del src, dst
    return r


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: this "
              "build runs the hot path on a single MI355X (the sharding design is described "
              "but not run)", file=sys.stderr)
        return 2
    import torch

    import sparse_attention_relu_amd as dsa
    import workloads as W

    dsa.load()
    torch.cuda.set_device(0)
    reps = args.cold_reps
    if args.only == "copy":
        print(json.dumps({"only": "copy", **copy_bandwidth(256, 5)}), flush=True)
        return 0
    if args.only in ("decode", "ragged"):
        wl = W.config(2 if args.only == "decode" else 3)
        r = bench_decode(dsa, wl, max(args.steps, 200 if args.only == "decode" else 100),
                         max(args.warmup, 10), reps or 50)
        print(json.dumps({"only": args.only, **r}), flush=True)
        return 0
    if args.only == "extend":
        wl = W.config(4)
        r = bench_extend_workload(dsa, wl, max(2, args.steps // 2), min(args.warmup, 2),
                                  reps or 20)
        print(json.dumps({"only": "extend", **r}), flush=True)
        return 0

    _log("long-context workload: generating")
    wl5 = W.config(5)
    _log("long-context workload: timing")
    lng = bench_extend_workload(dsa, wl5, args.steps, args.warmup, reps or 20)
    main_step = lng["steps"]["locality"]
    result = {
        "metric": METRIC,
        "value": main_step["ms_per_layer"],
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_step["ms_per_step"],
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl5.name, "seqs": wl5.S, "kv_len": int(wl5.seq_lens.max()),
                   "chunk_tokens": lng["T"], "page_size": wl5.PS, "index_topk": wl5.k,
                   "indexer_heads": wl5.H_idx, "indexer_dim": wl5.D_idx,
                   "mla_heads": wl5.H_mla, "dk": DK, "dv": DV, "layers": lng["layers"],
                   "indexshare": "1 full + 3 shared", "attend_feed": "locality selection",
                   "attend_path": main_step["path"],
                   "step": "4 layers: self-write; full layer indexer top-k + union (sizes "
                           "only when per query); "
                           "sparse MLA attention on the planned path"},
        "roofline": lng["roofline"],
        "long_extend": lng,
    }
    if args.only == "all":
        del wl5
        # the decode steps take tens of microseconds: time enough of them
        # (a few milliseconds) that host and box noise average out
        _log("decode batch")
        result["decode_batch"] = bench_decode(dsa, W.config(2), max(200, 2 * args.steps),
                                              max(20, args.warmup), reps or 50)
        _log("ragged decode")
        result["ragged_decode"] = bench_decode(dsa, W.config(3), max(100, 2 * args.steps),
                                               max(10, args.warmup), reps or 50)
        _log("chunked extend")
        result["chunked_extend"] = bench_extend_workload(dsa, W.config(4), max(4, args.steps),
                                                         args.warmup, reps or 20)
        result["copy_kernel"] = copy_bandwidth()
    if not args.no_cpu_baseline:
        _log("cpu baseline")
        result["cpu_baseline"] = cpu_baseline(W.config(5, layers=4), args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
