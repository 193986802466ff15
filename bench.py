#!/usr/bin/env python3
"""Benchmark of the DeepSeek-Sparse-Attention hot path on one MI355X.

One step = one DSA layer of the workload:
  decode  (default, 8 sequences x 8192 tokens): exact indexer top-k, then
          sparse absorbed-MLA decode over the selected positions;
  ragged decode (64 sequences, 4K..32K tokens, reported beside it);
  extend  (4 requests x (12288 + 1024), reported beside it): indexer top-k,
          query-block union tables, query-block sparse MLA.
Inputs are seeded synthetic tensors already resident in HBM when the timed
region starts. Prints ONE JSON line (rank 0).

  python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--config 2]
                  [--ragged-config 3|0] [--extend-config 4|5|0] [--no-cpu-baseline]
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


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=2, choices=[1, 2, 3],
                   help="decode workload (1 tiny, 2 8x8192, 3 ragged 64x[4K,32K])")
    p.add_argument("--extend-config", type=int, default=4, choices=[0, 1, 4, 5],
                   help="extend workload measured beside it (0 = none)")
    p.add_argument("--ragged-config", type=int, default=3, choices=[0, 3],
                   help="ragged decode workload reported beside it (0 = none)")
    p.add_argument("--long-config", type=int, default=5, choices=[0, 5],
                   help="long-context extend with IndexShare layers (0: skip)")
    p.add_argument("--qb", type=int, default=256, help="query block of the extend layer")
    p.add_argument("--only", choices=["all", "decode", "ragged", "extend", "long", "copy"],
                   default="all",
                   help="run one workload alone (for per-workload profiles); 'copy' times a "
                        "plain 256 MiB device copy, the scale of the HBM byte counters")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    return p.parse_args(argv)


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def _dev_inputs(wl, bname, layers=1):
    import numpy as np
    import torch

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    b = wl.batches[bname]
    return dict(
        page_table=i32(wl.page_table), seq_lens=i32(wl.seq_lens), cu=i32(b.cu_q_lens),
        idx_cache=wl.idx_cache.to_torch("cuda"),
        kv_cache=[wl.kv_cache[i].to_torch("cuda") for i in range(layers)],
        q_idx=bf16(b.q_idx), w=torch.from_numpy(b.w).cuda(),
        q=[bf16(b.q_mla[i]) for i in range(layers)],
        max_q_len=int(np.diff(b.cu_q_lens).max()),
    )


def _row_valid_counts(wl, cu):
    """n_valid per packed row (positions j < kv and j <= abs_q)."""
    import numpy as np

    T = int(cu[-1])
    n = np.zeros(T, dtype=np.int64)
    for s in range(wl.S):
        q0, q1 = int(cu[s]), int(cu[s + 1])
        a = int(wl.seq_lens[s]) - (q1 - q0) + np.arange(q1 - q0)
        n[q0:q1] = np.clip(np.minimum(a + 1, int(wl.seq_lens[s])), 0, None)
    return n


def _timed(step, steps, warmup):
    """Average ms per step over `steps` calls, events on the current stream."""
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


def _kernel_times(dsa, step, steps):
    """Per-kernel average launch duration (ms) from the library's event timer."""
    import torch

    torch.cuda.synchronize()
    dsa.profile_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    prof = dsa.profile_read()
    dsa.profile_enable(False)
    return {k: (n, tot / n) for k, (n, tot) in prof.items()}


def _kernel_times_cold(dsa, step, steps):
    """The same per-kernel durations with the caches cold: a 1 GiB buffer
    (four times the 256 MB infinity cache) is read before every step, outside
    the library's timed launches. Reading, not writing, leaves the caches
    holding clean lines, so the next kernel pays no write-back of the flush."""
    import torch

    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    dsa.profile_enable(True)
    for _ in range(steps):
        torch.sum(flush, dim=0, out=sink)  # a torch kernel: not one of the library's timed launches
        step()
    torch.cuda.synchronize()
    prof = dsa.profile_read()
    dsa.profile_enable(False)
    del flush
    return {k: (n, tot / n) for k, (n, tot) in prof.items()}


def _roofline_entry(bound, work, ms, per_step_launches=1):
    """work = algorithmic bytes (hbm) or flops (mfma) of ONE launch."""
    if bound == "hbm":
        achieved = work / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    achieved = work / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}


# Sources whose text decides each kernel's machine code.
KERNEL_SOURCES = {
    "idx_score_stream": "indexer.hip", "idx_score_flat": "indexer.hip",
    "idx_score_tiles": "indexer.hip",
    "topk_select": "indexer.hip", "mla_decode_partial": "mla.hip",
    "mla_decode_combine": "mla.hip", "mla_decode_combine_wide": "mla.hip",
    "mla_extend_qblock": "mla.hip",
    "union_clear": "union.hip", "union_mark": "union.hip", "union_compact": "union.hip",
    "union_member": "union.hip", "page_pool": "indexer.hip", "page_token_list": "indexer.hip",
    "paged_write_rows": "cache_write.hip",
}


def kernel_source_hash(kernel):
    """sha256 over the kernel's source file and the shared device header."""
    import hashlib

    csrc = os.path.join(ROOT, "sparse_attention_relu_amd", "csrc")
    h = hashlib.sha256()
    for name in (KERNEL_SOURCES[kernel], "common.h"):
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


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------
def bench_decode(dsa, wl, args):
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

    ms = _timed(step, args.steps, args.warmup)
    kt = _kernel_times(dsa, step, args.steps)
    kt_cold = _kernel_times_cold(dsa, step, max(5, args.steps // 5))

    # algorithmic work per launch
    nval = _row_valid_counts(wl, b.cu_q_lens)
    sel = topk.cpu().numpy()
    n_sel = int((sel >= 0).sum())
    D, Hi, PS = wl.D_idx, wl.H_idx, wl.PS
    score_bytes = (int(nval.sum()) * (D * 2 + 4) + T * Hi * (D * 2 + 4)
                   + int(np.ceil(nval / PS).sum()) * 4)
    work = {
        "idx_score_stream": ("hbm", score_bytes),
        "idx_score_flat": ("hbm", score_bytes),
        "topk_select": ("hbm", int(nval.sum()) * 4 + T * k * 4),
        "mla_decode_partial": ("hbm", n_sel * DK * 2 + T * k * 4 + T * H * DK * 2),
        "mla_decode_combine": ("hbm", T * H * DV * 2),
    }
    kernels = {}
    for name, (n, avg) in kt.items():
        bound, w = work.get(name, ("hbm", 0))
        e = {"avg_us": round(avg * 1e3, 2), "launches_per_step": n // args.steps}
        if w:
            e.update(_roofline_entry(bound, w, avg))
            e["work"] = w
        if name in kt_cold:
            c = {"avg_us": round(kt_cold[name][1] * 1e3, 2)}
            if w:
                c["frac"] = _roofline_entry(bound, w, kt_cold[name][1])["frac"]
            e["cold"] = c
        kernels[name] = e
    dom = max(kt, key=lambda nm: kt[nm][1] * kt[nm][0])
    bound, w = work[dom]
    roof = _roofline_entry(bound, w, kt[dom][1])
    roof.update({"kernel": dom, "traffic": measured_traffic(dom, wl.name),
                 "work_per_launch": w, "avg_launch_us": round(kt[dom][1] * 1e3, 2)})

    def part(names):
        return sum(kt[nm][1] * kt[nm][0] for nm in names if nm in kt) / args.steps

    return dict(ms=ms, tok_s=T / (ms * 1e-3), kernels=kernels, roofline=roof,
                selected=n_sel, keys=int(nval.sum()),
                indexer_ms=round(part(("idx_score_stream", "idx_score_flat", "topk_select")), 4),
                attend_ms=round(part(("mla_decode_partial", "mla_decode_combine")), 4))


def bench_page_decode(dsa, wl, args):
    """The same decode layer with page-level selection: the page top-k
    (k_pages = k / PS pages, max-pooled page scores), then sparse MLA over
    every valid position of those pages (page lists read directly)."""
    import torch

    d = _dev_inputs(wl, "decode")
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

    steps = max(5, args.steps // 2)
    ms = _timed(step, steps, min(args.warmup, 3))
    kt = _kernel_times(dsa, step, steps)
    return {"k_pages": kp, "ms_per_step": round(ms, 5), "tok_s": round(T / (ms * 1e-3), 1),
            "kernels_us": {nm: round(avg * 1e3, 2) for nm, (n, avg) in kt.items()}}


# ----------------------------------------------------------------------------
# extend
# ----------------------------------------------------------------------------
def bench_extend(dsa, wl, args, QB, steps=None):
    import numpy as np
    import torch

    layers = len(wl.kv_cache)
    d = _dev_inputs(wl, "extend", layers=layers)
    b = wl.batches["extend"]
    T, k, H = b.T, wl.k, wl.H_mla
    u_max = wl.u_max
    nqb = (T + QB - 1) // QB
    topk = torch.empty((T, k), dtype=torch.int32, device="cuda")
    units = torch.empty((nqb, u_max), dtype=torch.int32, device="cuda")
    counts = torch.empty((nqb,), dtype=torch.int32, device="cuda")
    member = torch.empty((nqb, u_max, QB), dtype=torch.uint64, device="cuda")
    outs = [torch.empty((T, H, DV), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    ws_i = torch.empty(dsa.indexer_topk_workspace(T, wl.S, wl.H_idx, wl.D_idx, wl.PS, wl.MP, k,
                                                  d["max_q_len"]), dtype=torch.uint8,
                       device="cuda")
    ws_u = torch.empty(max(1, dsa.block_union_workspace(T, wl.S, wl.MP, QB, u_max)),
                       dtype=torch.uint8, device="cuda")

    # IndexShare: the first layer is full (indexer + union), the others are
    # shared and attend with its tables (one slot)
    full_slot, src_slot, n_full = dsa.index_share_map(["full"] + ["shared"] * (layers - 1))
    assert n_full == 1

    def step():
        for i in range(layers):
            if i in full_slot:
                dsa.indexer_topk(d["q_idx"], d["w"], d["idx_cache"], d["page_table"],
                                 d["seq_lens"], d["cu"], k, d["max_q_len"], out=topk,
                                 workspace=ws_i)
                dsa.block_union(topk, d["seq_lens"], d["cu"], wl.PS, wl.MP, QB, u_max,
                                out=(units, counts, member), workspace=ws_u)
            dsa.sparse_mla_extend(d["q"][i], d["kv_cache"][i], d["page_table"], d["seq_lens"],
                                  d["cu"], units, counts, member, QB, wl.sm_scale, out=outs[i])

    steps = steps or max(2, args.steps // 4)
    ms = _timed(step, steps, min(args.warmup, 2))
    kt = _kernel_times(dsa, step, steps)
    cnt = counts.cpu().numpy()
    sel = topk.cpu().numpy()
    nval = _row_valid_counts(wl, b.cu_q_lens)
    exec_flops = int(np.minimum(cnt, u_max).sum()) * QB * H * wl.PS * (DK + DV) * 2
    useful_flops = int((sel >= 0).sum()) * H * (DK + DV) * 2
    idx_flops = 2 * wl.H_idx * wl.D_idx * int(nval.sum())
    work = {
        "idx_score_tiles": ("mfma", idx_flops),
        "topk_select": ("hbm", int(nval.sum()) * 4 + T * k * 4),
        "mla_extend_qblock": ("mfma", exec_flops),
        "union_member": ("hbm", T * k * 4 + nqb * u_max * QB * 8),
        "union_mark": ("hbm", T * k * 4),
    }
    kernels = {}
    for name, (n, avg) in kt.items():
        e = {"avg_us": round(avg * 1e3, 2), "launches_per_step": n // steps}
        if name in work:
            bound, w = work[name]
            e.update(_roofline_entry(bound, w, avg))
            e["work"] = w
        kernels[name] = e
    # redundant-fetch ratios: per-query pages vs block unions vs distinct pages
    seq, _ = _rows_seq(wl, b.cu_q_lens)
    keys = np.where(sel >= 0, seq[:, None] * wl.MP + sel // wl.PS, -1)
    per_query_pages = sum(len(np.unique(r[r >= 0])) for r in keys)
    distinct = len(np.unique(keys[keys >= 0]))
    res = dict(ms_per_step=round(ms, 4), layers=layers, QB=QB,
               ms_full_layer=round(ms - (layers - 1) * kt["mla_extend_qblock"][1], 4)
               if layers > 1 else round(ms, 4),
               ms_shared_layer=round(kt["mla_extend_qblock"][1], 4),
               indexer_ms=round(kt.get("idx_score_tiles", (0, 0))[1]
                                + kt.get("topk_select", (0, 0))[1], 4),
               union_per_block={"min": int(cnt.min()), "mean": round(float(cnt.mean()), 1),
                                "max": int(cnt.max())},
               redundant_fetch={"per_query": round(per_query_pages / max(distinct, 1), 1),
                                "qblock": round(float(cnt.sum()) / max(distinct, 1), 2)},
               mfma_executed_tflop=round(exec_flops / 1e12, 3),
               mfma_useful_tflop=round(useful_flops / 1e12, 3),
               kernels=kernels)
    dom = max(kt, key=lambda nm: kt[nm][1] * kt[nm][0])
    if dom in work:
        bound, w = work[dom]
        roof = _roofline_entry(bound, w, kt[dom][1])
        roof.update({"kernel": dom, "traffic": measured_traffic(dom, wl.name),
                     "work_per_launch": w, "avg_launch_us": round(kt[dom][1] * 1e3, 2)})
        res["roofline"] = roof
    res["per_query"] = _per_query_attend(dsa, wl, d, topk, outs, steps, kt)
    # the library's own choice between the two paths for these unions, and
    # the step with the chosen path for every layer (indexer and union once)
    res["attend_path_chosen"] = dsa.extend_attend_path(cnt, T, H, k, wl.PS, QB, u_max)
    per_layer = (res["per_query"]["ms_per_layer"] if res["attend_path_chosen"] == "per_query"
                 else kt["mla_extend_qblock"][1])
    res["ms_per_step_chosen_path"] = round(ms - layers * kt["mla_extend_qblock"][1]
                                           + layers * per_layer, 4)
    res["cache_write"] = _cache_write(dsa, wl, d, steps)
    return res


def _cache_write(dsa, wl, d, steps):
    """The self-write of the chunk's new tokens ahead of the layer: indexer
    keys (one call) and latent rows (c_kv, k_rope). Timed last: it rewrites
    the chunk's own cache slots."""
    import torch

    T = int(d["cu"][-1].item())
    g = torch.Generator(device="cuda").manual_seed(11)
    keys = torch.randint(-2, 3, (T, wl.D_idx), generator=g, device="cuda").to(torch.bfloat16)
    lat = torch.randn((T, DK), generator=g, device="cuda").to(torch.bfloat16)

    def step():
        dsa.paged_write(keys, d["idx_cache"], d["page_table"], d["seq_lens"], d["cu"])
        dsa.paged_write(lat[:, :DV], d["kv_cache"][0], d["page_table"], d["seq_lens"], d["cu"])
        dsa.paged_write(lat[:, DV:], d["kv_cache"][0], d["page_table"], d["seq_lens"], d["cu"],
                        col0=DV)

    step()
    kt = _kernel_times(dsa, step, steps)
    n, avg = kt["paged_write_rows"]
    ms = avg * n / steps  # device time of the three writes (the host calls take longer)
    moved = T * (wl.D_idx + DK) * 2 * 2  # read and written once
    return {"tokens": T, "launches": n // steps, "us_per_layer": round(ms * 1e3, 2),
            "roofline": _roofline_entry("hbm", moved, ms)}


def _per_query_attend(dsa, wl, d, topk, outs, steps, kt_qblock):
    """The same layers attended per query: each packed row gathers its own
    selected latent rows (the decode kernels run on the extend batch), with no
    block union. Reported beside the query-block kernel; its outputs are
    compared with the query-block outputs of the same selections."""
    import torch

    layers = len(outs)
    T, k, H = topk.shape[0], topk.shape[1], outs[0].shape[1]
    ws_d = torch.empty(max(1, dsa.sparse_mla_decode_workspace(T, H, k)), dtype=torch.uint8,
                       device="cuda")
    outs_pq = [torch.empty_like(o) for o in outs]

    def step():
        for i in range(layers):
            dsa.sparse_mla_decode(d["q"][i], d["kv_cache"][i], d["page_table"], d["seq_lens"],
                                  d["cu"], topk, wl.sm_scale, out=outs_pq[i], workspace=ws_d)

    ms = _timed(step, steps, 1)
    kt = _kernel_times(dsa, step, steps)
    torch.cuda.synchronize()
    diff = max(float((a.float() - b.float()).abs().max()) for a, b in zip(outs, outs_pq))
    n_sel = int((topk >= 0).sum())
    gather = n_sel * DK * 2 + T * k * 4 + T * H * DK * 2
    part = kt["mla_decode_partial"][1]
    e = {"ms_per_layer": round(ms / layers, 4),
         "partial_us": round(part * 1e3, 2),
         "combine_us": round(kt["mla_decode_combine"][1] * 1e3, 2),
         "partial_roofline": _roofline_entry("hbm", gather, part),
         "gathered_bytes_per_layer": gather,
         "speedup_vs_qblock": round(kt_qblock["mla_extend_qblock"][1] / (ms / layers), 2),
         "max_abs_diff_vs_qblock": round(diff, 5)}
    return e


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


# ----------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ----------------------------------------------------------------------------
def cpu_baseline(wl, seconds):
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    from workloads import bf16_to_f64

    b = wl.batches["decode"]
    q_idx = bf16_to_f64(b.q_idx)
    w = b.w.astype(np.float64)
    icache = wl.idx_cache.f64_view()
    kv = wl.kv_cache[0].f64_view()
    q = bf16_to_f64(b.q_mla[0])
    rows_done = 0
    t0 = time.perf_counter()
    t_end = t0 + seconds
    r = 0
    while True:
        rows = [r % b.T]
        tk = oracle.indexer_topk(q_idx, w, icache, wl.page_table, wl.seq_lens, b.cu_q_lens, wl.k,
                                 rows=rows)
        oracle.sparse_mla(q, kv, wl.page_table, wl.seq_lens, b.cu_q_lens, tk, wl.sm_scale, wl.Dv,
                          rows=rows)
        rows_done += 1
        r += 1
        if time.perf_counter() >= t_end and rows_done >= 1:
            break
    dt = time.perf_counter() - t0
    threads = 0
    for info in threadpool_info():
        if info.get("user_api") == "blas":
            threads = max(threads, int(info.get("num_threads", 0)))
    return {"value": round(rows_done / dt, 3), "unit": "tok/s", "cores": max(threads, 1),
            "kind": "oracle",
            "sample": f"{rows_done} decode rows (indexer top-k + sparse MLA, fp64 NumPy) of the "
                      f"{wl.name} workload in {dt:.1f} s"}


# ----------------------------------------------------------------------------
def copy_calibration(mib=256, reps=5):
    """A plain device copy of known size: under a counter profiler its
    FETCH_SIZE / WRITE_SIZE per dispatch give the counters' byte scale."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"only": "copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "ms": round(ms, 4), "GB_s": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}),
          flush=True)
    return 0


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path runs on a single MI355X here)", file=sys.stderr)
        return 2
    import torch

    import sparse_attention_relu_amd as dsa
    import workloads as W

    dsa.load()
    torch.cuda.set_device(0)
    if args.only == "copy":
        return copy_calibration()
    if args.only in ("ragged", "extend", "long"):  # one side workload alone, its own line
        if args.only == "long":
            wll = W.config(args.long_config or 5)
            line = bench_extend(dsa, wll, args, 256, steps=max(2, args.steps // 10))
            line["workload"] = wll.name
        elif args.only == "ragged":
            wlr = W.config(args.ragged_config or 3)
            rd = bench_decode(dsa, wlr, args)
            line = {"workload": wlr.name, "tok_s": round(rd["tok_s"], 1),
                    "ms_per_step": round(rd["ms"], 5), "roofline": rd["roofline"],
                    "kernels": rd["kernels"], "page_decode": bench_page_decode(dsa, wlr, args)}
        else:
            wle = W.config(args.extend_config or 4)
            qb = args.qb if args.qb in wle.QB else wle.QB[0]
            line = bench_extend(dsa, wle, args, qb)
            line["workload"] = wle.name
        print(json.dumps({"only": args.only, **line}), flush=True)
        return 0
    wl = W.config(args.config)
    dec = bench_decode(dsa, wl, args)
    result = {
        "metric": METRIC,
        "value": round(dec["tok_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "seqs": wl.S, "kv_len": int(wl.seq_lens.max()),
                   "page_size": wl.PS, "index_topk": wl.k, "indexer_heads": wl.H_idx,
                   "indexer_dim": wl.D_idx, "mla_heads": wl.H_mla, "dk": DK, "dv": DV,
                   "step": "one DSA decode layer: indexer top-k + sparse MLA"},
        "roofline": dec["roofline"],
        "kernels": dec["kernels"],
        "page_decode": bench_page_decode(dsa, wl, args),
    }
    if args.only == "all" and args.ragged_config and args.ragged_config != args.config:
        wlr = W.config(args.ragged_config)
        rd = bench_decode(dsa, wlr, args)
        result["ragged_decode"] = {
            "workload": wlr.name, "seqs": wlr.S, "tokens": int(wlr.seq_lens.sum()),
            "tok_s": round(rd["tok_s"], 1), "ms_per_step": round(rd["ms"], 5),
            "indexer_ms": rd["indexer_ms"], "attend_ms": rd["attend_ms"],
            "roofline": rd["roofline"], "kernels": rd["kernels"],
            "page_decode": bench_page_decode(dsa, wlr, args)}
    if args.only == "all" and args.extend_config:
        wle = W.config(args.extend_config)
        qb = args.qb if args.qb in wle.QB else wle.QB[0]
        ext = bench_extend(dsa, wle, args, qb)
        ext["workload"] = wle.name
        result["extend"] = ext
    if args.only == "all" and args.long_config:
        wll = W.config(args.long_config)
        lng = bench_extend(dsa, wll, args, 256, steps=max(2, args.steps // 10))
        lng["workload"] = wll.name
        result["long_extend"] = lng
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
