#!/usr/bin/env python3
"""Decode-step benchmark of the context-sparse decode path on one MI355X.

A step is one attention layer of sparse decode for the whole batch: the exact
top-k indexer (score pass + radix select) followed by the gather-attend over the
selected rows (plus the one-token cache append on workloads that grow).  The
dense decode of the same layer is timed the same way for comparison.  Inputs are
seeded synthetic bf16 caches already resident in HBM when timing starts.

Prints ONE JSON line: steps/s (value), the per-kernel roofline of the dominant
launch group (the indexer) against the 8 TB/s HBM peak, and the fp64 CPU oracle
timed on the host as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode steps/s + effective HBM GB/s (% of peak) at 50x sparsity vs dense"
PEAK_HBM_BPS = 8.0e12          # MI355X HBM3E peak
FLUSH_BYTES = 1 << 30          # written before a cold launch: flushes the 256 MB Infinity Cache and the L2s


def traffic_file(cfg):
    return os.path.join(ROOT, "profiles", f"traffic_index_topk_C{cfg}.txt")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", type=int, default=5,
                    help="decode configuration 1-5 (default 5, the agentic ragged batch: the largest 50x workload)")
    ap.add_argument("--ratio", type=int, default=50, help="sparsity N/k (default 50)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip timing each launch group after a 1 GiB cache flush")
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph",
                    help="replay captured HIP graphs (default) or launch eagerly from Python")
    ap.add_argument("--quest", action="store_true",
                    help="also time the Quest-style page selection step (current-page summary update, page "
                         "selection, attend over the pages' tokens) at the same token budget, with its recall "
                         "of the exact top-k")
    ap.add_argument("--labels", action="store_true",
                    help="also time the lightweight indexer on 16-channel label rows (current-page label "
                         "update, label index, attend), with its recall of the exact top-k")
    ap.add_argument("--sampled", action="store_true",
                    help="also time the stochastic step (top-k/2 plus k/2 uniform draws from the rest)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB 3 times (a plain device copy of known "
                         "size, the reference for scaling memory-traffic counters)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="no benchmark: summarise the rocprofv3 output under DIR (kernel trace, and counters "
                         "when collected) of an earlier run of this script, per kernel, warm and cold")
    return ap.parse_args()


def algorithmic_bytes(seq_lens, kps, B, hq, hkv):
    """Bytes each piece must move at minimum (bf16 rows of 256 B)."""
    n = np.asarray(seq_lens, np.int64)
    k = np.asarray(kps, np.int64)
    q_bytes = B * hq * 128 * 2
    out_bytes = B * hq * 128 * 4
    index = int((hkv * n * 256).sum() + q_bytes + (hq * k * 4).sum())
    attend = int((hq * k * (512 + 4)).sum() + q_bytes + out_bytes)
    dense = int((hkv * n * 512).sum() + q_bytes + out_bytes)
    return index, attend, dense


def read_traffic(cfg):
    """HBM bytes per launch of the indexer from the committed counter summary, if any."""
    path = traffic_file(cfg)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            key, val = line.split(":", 1)
            vals[key.strip()] = val.strip()
    try:
        return float(vals["hbm_bytes_per_launch"]) if vals.get("kernel_source_sha") == source_sha() else None
    except (KeyError, ValueError):
        return None


def source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("index_topk.hip", "sdi_device.hpp", "sdi_radix.hpp", "sdi_index.hpp"):
        h.update(open(os.path.join(ROOT, "sparse_attention_decode_index_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def trace_summary(root):
    """Per-kernel durations from a rocprofv3 kernel trace (CSV) of a run of this script:
    warm launches, and cold ones -- the first launch of each library kernel after a
    1 GiB cache-flush fill (torch's uint8 FillFunctor taking over 50 us).  With counter
    collection output present, the counters per dispatch as well."""
    import csv
    import glob
    import statistics as st
    traces = sorted(glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True))
    if not traces:
        sys.exit(f"no *kernel_trace.csv under {root}")
    rows = []
    for path in traces:
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()

    def short(name):
        name = name.split("(")[0] if name.startswith("void ") else name
        return name.replace("void ", "")

    warm, cold = {}, {}
    seen = None                                  # library kernels met since the last flush
    for t0, t1, name in rows:
        us = (t1 - t0) / 1e3
        if "FillFunctor<unsigned char>" in name and us > 50.0:
            seen = set()
            continue
        if "sdi::" not in name:
            continue
        k = short(name)
        if seen is not None and k not in seen:   # the first launch of this kernel after a flush
            seen.add(k)
            cold.setdefault(k, []).append(us)
        else:
            warm.setdefault(k, []).append(us)
    out = {"kernels": {}}
    for k in sorted(set(warm) | set(cold), key=lambda n: -sum(warm.get(n, [0.0]))):
        v = warm.get(k, [])
        e = {"calls": len(v), "avg_us": st.mean(v), "min_us": min(v), "max_us": max(v)} if v else {"calls": 0}
        c = cold.get(k, [])
        if c:
            e.update({"cold_calls": len(c), "cold_avg_us": st.mean(c), "cold_median_us": st.median(c)})
        out["kernels"][k] = e
    counters = sorted(glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True))
    if counters:
        per = {}
        for path in counters:
            with open(path) as f:
                for r in csv.DictReader(f):
                    name = short(r.get("Kernel_Name", ""))
                    key = (name, r.get("Counter_Name", ""))
                    per.setdefault(key, {}).setdefault(r.get("Dispatch_Id", ""), 0.0)
                    per[key][r.get("Dispatch_Id", "")] += float(r.get("Counter_Value", 0.0))
        out["counters_per_dispatch_kib"] = {
            f"{n} {c}": {"dispatches": len(d), "mean": st.mean(d.values()), "min": min(d.values()),
                         "max": max(d.values())} for (n, c), d in sorted(per.items())}
    print(json.dumps(out, indent=1))


def cpu_baseline(wl, target_s):
    """The fp64 oracle (untuned) on the host over the same workload: whole decode steps
    (scores, exact top-k, attend) of the first `nb` sequences, nb doubling until the
    sample takes a few seconds, then repeated up to about `target_s`; steps/s is scaled
    to the full batch."""
    import oracle

    def run(nb):
        cache = oracle.Cache(wl.k_cache, wl.v_cache, wl.page_table[:nb], wl.seq_lens[:nb], wl.num_kv_heads)
        kps = wl.k_per_seq()[:nb]
        t0 = time.perf_counter()
        oracle.decode_step(cache, wl.q[:nb], kps, int(wl.k_max()))
        return time.perf_counter() - t0

    nb, t = 1, run(1)
    while nb < wl.batch and t < target_s / 4:
        nb = min(wl.batch, nb * 2)
        t = run(nb)
    reps, total = 1, t
    while total + t <= target_s:
        total += run(nb)
        reps += 1
    per_step = total / reps * wl.batch / nb
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": 1.0 / per_step, "unit": "decode steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": cpu_model,
            "sample": f"{reps} x the oracle's decode step (fp64 scores, exact top-k, attend) on {nb} of "
                      f"{wl.batch} sequences ({total:.1f} s), scaled to the whole batch"}


def quest_leg(sdi, wl, kv_full, step_args, timed_graph, per, reps, n_q, k_max, idx, out, ws_attend, dense_s):
    """Quest-style step at the exact indexer's token budget: the current pages'
    summaries refreshed, the page selection (m_b = ceil(k_b / 16) pages, current page
    included), then the gather-attend over those pages' tokens (16 m_b entries per
    row).  Recall = share of the exact top-k tokens (step 0) that the selected pages
    contain."""
    import torch
    dev = idx.device
    B, hq = wl.batch, wl.num_q_heads
    pages_max = (k_max + 15) // 16
    budget = {}
    for j in range(n_q):
        kps = step_args(j)[2]
        if id(kps) not in budget:
            m = (kps + 15) // 16
            budget[id(kps)] = (m, 16 * m)
    summary = sdi.quest_summarize(kv_full)                   # prefill: every page once
    qidx = torch.empty((B, hq, 16 * pages_max), dtype=torch.int32, device=dev)
    ws_q = torch.empty(max(1, sdi.load_library().sparse_decode_quest_select_workspace(
        ctypes.byref(kv_full.struct()), hq, pages_max)), dtype=torch.uint8, device=dev)
    ws_qa = torch.empty(max(1, sdi.attend_workspace_bytes(kv_full, hq, 16 * pages_max)), dtype=torch.uint8,
                        device=dev)

    def update(s):
        kv, _, _ = step_args(s)
        sdi.quest_summarize(kv, summary, current_pages_only=True, stream=torch.cuda.current_stream())

    def select(s):
        kv, q, kps = step_args(s)
        sdi.quest_select(kv, q, summary, budget[id(kps)][0], pages_max, idx_out=qidx, workspace=ws_q,
                         stream=torch.cuda.current_stream())

    def attend(s):
        kv, q, kps = step_args(s)
        sdi.attend(kv, q, qidx, budget[id(kps)][1], out=out, workspace=ws_qa, stream=torch.cuda.current_stream())

    def step(s):
        update(s)
        select(s)
        attend(s)

    for s in range(3):
        step(s)
    torch.cuda.synchronize()
    t_upd, _ = timed_graph(update, max(1, reps), per)
    t_sel, _ = timed_graph(select, max(1, reps), per)
    t_att, _ = timed_graph(attend, max(1, reps), per)
    t_step, _ = timed_graph(step, max(1, reps), per)
    # recall of the exact selection, step 0
    kv, q, kps = step_args(0)
    sdi.index_topk(kv, q, kps, k_max, idx_out=idx)
    select(0)
    torch.cuda.synchronize()
    ex, qt = idx.cpu().numpy(), qidx.cpu().numpy()
    rec = []
    for b in range(B):
        for h in range(hq):
            e = ex[b, h][ex[b, h] >= 0]
            if len(e):
                rec.append(np.isin(e, qt[b, h]).mean())
    res = {"pages_max": pages_max, "tokens_max": 16 * pages_max, "summary_update_us": t_upd * 1e6,
           "select_us": t_sel * 1e6, "attend_us": t_att * 1e6, "step_us": t_step * 1e6,
           "recall_of_exact_topk": float(np.mean(rec)),
           "select_bytes_per_launch": int((wl.num_kv_heads * ((wl.seq_lens.astype(np.int64) + 15) // 16) * 512).sum())}
    if dense_s is not None:
        res["speedup_vs_dense"] = dense_s / t_step
    return res


def calibrate_channels(wl, r=16, sample=2048):
    """Offline channel choice for the label indexer: per kv head the r channels of
    largest mean |K| over the first `sample` tokens of sequence 0 (a calibration
    sample, not the step's data)."""
    n = min(sample, int(wl.seq_lens[0]))
    pages = wl.page_table[0, :-(-n // 16)]
    vals = (wl.k_cache[pages].astype(np.uint32) << 16).view(np.float32)    # only the sample's pages
    ch = np.zeros((wl.num_kv_heads, r), np.int32)
    for g in range(wl.num_kv_heads):
        rows = vals[:, g].reshape(-1, 128)[:n]
        ch[g] = np.sort(np.argsort(-np.abs(rows).mean(axis=0), kind="stable")[:r])
    return ch


def labels_leg(sdi, wl, kv_full, step_args, timed_graph, per, reps, k_max, idx, out, ws_index, ws_attend,
               dense_s):
    """Lightweight-indexer step at the same k: the current pages' label rows refreshed,
    the top-k of the 16-channel scores, then the gather-attend.  Recall = share of the
    exact top-k tokens (step 0) that the label indexer also selects."""
    import torch
    dev = idx.device
    ch = torch.from_numpy(calibrate_channels(wl)).to(dev)
    labels = sdi.label_build(kv_full, ch)                    # prefill: every page once
    lidx = torch.empty_like(idx)

    def update(s):
        kv, _, _ = step_args(s)
        sdi.label_build(kv, ch, labels, current_pages_only=True, stream=torch.cuda.current_stream())

    def index(s):
        kv, q, kps = step_args(s)
        sdi.label_index_topk(kv, q, labels, ch, kps, k_max, idx_out=lidx, workspace=ws_index,
                             stream=torch.cuda.current_stream())

    def attend(s):
        kv, q, kps = step_args(s)
        sdi.attend(kv, q, lidx, kps, out=out, workspace=ws_attend, stream=torch.cuda.current_stream())

    def step(s):
        update(s)
        index(s)
        attend(s)

    for s in range(3):
        step(s)
    torch.cuda.synchronize()
    t_upd, _ = timed_graph(update, max(1, reps), per)
    t_idx, _ = timed_graph(index, max(1, reps), per)
    t_att, _ = timed_graph(attend, max(1, reps), per)
    t_step, _ = timed_graph(step, max(1, reps), per)
    kv, q, kps = step_args(0)
    sdi.index_topk(kv, q, kps, k_max, idx_out=idx)
    index(0)
    torch.cuda.synchronize()
    ex, lt = idx.cpu().numpy(), lidx.cpu().numpy()
    rec = []
    for b in range(wl.batch):
        for h in range(wl.num_q_heads):
            e = ex[b, h][ex[b, h] >= 0]
            if len(e):
                rec.append(np.isin(e, lt[b, h]).mean())
    n = wl.seq_lens.astype(np.int64)
    res = {"channels": 16, "label_update_us": t_upd * 1e6, "index_us": t_idx * 1e6, "attend_us": t_att * 1e6,
           "step_us": t_step * 1e6, "recall_of_exact_topk": float(np.mean(rec)),
           "index_bytes_per_launch": int((wl.num_kv_heads * n * 32).sum())}
    if dense_s is not None:
        res["speedup_vs_dense"] = dense_s / t_step
    return res


def sampled_leg(sdi, wl, kv_full, step_args, timed_graph, per, reps, n_q, k_max, idx, out, ws_index, dense_s):
    """Stochastic step at the same total budget k: the exact top-ceil(k/2), floor(k/2)
    uniform draws from the remaining tokens (each weighted by the remaining count over
    the draws), then the two-list attend.  The draws are inputs, made once on the host
    and resident like the queries.  Quality on this data: the mean relative L2 error of
    the output against dense decode, for this estimate and for exact top-k at budget k."""
    import torch
    dev = idx.device
    B, hq = wl.batch, wl.num_q_heads
    kd_max, s_max = (k_max + 1) // 2, max(1, k_max // 2)
    split = {}
    for j in range(n_q):
        kps = step_args(j)[2]
        if id(kps) not in split:
            split[id(kps)] = ((kps + 1) // 2, kps // 2)
    rng = np.random.default_rng(wl.seed + 7)
    draws = torch.from_numpy(rng.integers(0, 2 ** 32, size=(B, hq, s_max), dtype=np.uint64)
                             .astype(np.uint32).view(np.int32)).to(dev)
    kidx = torch.empty((B, hq, kd_max), dtype=torch.int32, device=dev)
    sample = torch.empty((B, hq, s_max), dtype=torch.int32, device=dev)
    weight = torch.empty((B, hq), dtype=torch.float32, device=dev)
    ws_s = torch.empty(max(1, sdi.attend_sampled_workspace_bytes(kv_full, hq, kd_max, s_max)), dtype=torch.uint8,
                       device=dev)

    def index(s):
        kv, q, kps = step_args(s)
        sdi.index_topk(kv, q, split[id(kps)][0], kd_max, idx_out=kidx, workspace=ws_index,
                       stream=torch.cuda.current_stream())

    def draw(s):
        kv, q, kps = step_args(s)
        kd, sv = split[id(kps)]
        sdi.sample_residual(kv, kidx, kd, draws, sv, sample_out=sample, weight_out=weight,
                            stream=torch.cuda.current_stream())

    def attend(s):
        kv, q, kps = step_args(s)
        kd, sv = split[id(kps)]
        sdi.attend_sampled(kv, q, kidx, kd, sample, weight, sv, out=out, workspace=ws_s,
                           stream=torch.cuda.current_stream())

    def step(s):
        index(s)
        draw(s)
        attend(s)

    for s in range(3):
        step(s)
    torch.cuda.synchronize()
    t_idx, _ = timed_graph(index, max(1, reps), per)
    t_smp, _ = timed_graph(draw, max(1, reps), per)
    t_att, _ = timed_graph(attend, max(1, reps), per)
    t_step, _ = timed_graph(step, max(1, reps), per)
    kv, q, kps = step_args(0)
    step(0)
    est = out.clone()
    sdi.index_topk(kv, q, kps, k_max, idx_out=idx)
    ex = sdi.attend(kv, q, idx, kps)
    dn = sdi.dense(kv, q)
    torch.cuda.synchronize()

    def rel(o):
        return float(((o - dn).norm(dim=-1) / dn.norm(dim=-1).clamp_min(1e-30)).mean())

    res = {"kept": "ceil(k/2)", "draws": "floor(k/2)", "index_us": t_idx * 1e6, "sample_us": t_smp * 1e6,
           "attend_us": t_att * 1e6, "step_us": t_step * 1e6,
           "rel_err_vs_dense": {"stochastic": rel(est), "exact_topk_k": rel(ex)}}
    if dense_s is not None:
        res["speedup_vs_dense"] = dense_s / t_step
    return res


def main():
    args = parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the sparse decode path here has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import sparse_attention_decode_index_amd as sdi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    wl = synth.config(args.config, ratio=args.ratio)
    B, hq, hkv = wl.batch, wl.num_q_heads, wl.num_kv_heads

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    k_cache, v_cache = bf16(wl.k_cache), bf16(wl.v_cache)
    page_table = torch.from_numpy(wl.page_table).to(dev)
    seq_lens = torch.from_numpy(wl.seq_lens).to(dev)
    total = args.warmup + args.steps
    growth = wl.steps > 1
    # a fresh query per step; growing workloads also append one token per step (and recompute k)
    n_q = min(total, 64) if not growth else min(total, wl.steps)
    qs = [bf16(synth.queries(wl.seed, s, B, hq)) for s in range(n_q)]
    appends, kps_steps, nmax_steps = [], [], []
    host = wl
    for s in range(n_q if growth else 1):
        kps_steps.append(torch.from_numpy(host.k_per_seq()).to(dev))
        nmax_steps.append(host.n_max)
        if growth and s + 1 < n_q:
            tok, pages, slots, kr, vr = host.new_rows()
            appends.append((torch.from_numpy(pages).to(dev), torch.from_numpy(slots).to(dev), bf16(kr), bf16(vr)))
            host.seq_lens = (host.seq_lens + 1).astype(np.int32)
    seq_lens_steps = None
    if growth:           # restore: the device cache starts at step 0
        host.seq_lens = (host.seq_lens - (n_q - 1)).astype(np.int32)
        seq_lens_steps = [torch.from_numpy((host.seq_lens + s).astype(np.int32)).to(dev) for s in range(n_q)]
    k_max = int(max(int(t.max().item()) for t in kps_steps))
    n_max_all = max(nmax_steps)
    kv_full = sdi.PagedKV(k_cache, v_cache, page_table, seq_lens, n_max=n_max_all)
    idx = torch.empty((B, hq, k_max), dtype=torch.int32, device=dev)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device=dev)
    ws_index = torch.empty(max(1, sdi.index_topk_workspace_bytes(kv_full, hq, k_max)), dtype=torch.uint8, device=dev)
    ws_attend = torch.empty(max(1, sdi.attend_workspace_bytes(kv_full, hq, k_max)), dtype=torch.uint8, device=dev)
    ws_dense = torch.empty(max(1, sdi.dense_workspace_bytes(kv_full, hq)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    stream = torch.cuda.current_stream()

    def step_args(s):
        j = s % n_q
        sl = seq_lens_steps[j] if growth else seq_lens
        kv = sdi.PagedKV(k_cache, v_cache, page_table, sl, n_max=nmax_steps[j] if growth else wl.n_max)
        return kv, qs[j], kps_steps[j if growth else 0]

    def run_step(s, ev=None):
        j = s % n_q
        if growth and j > 0:                              # a0: append this step's token (plain copies)
            pg, sl_, kr, vr = appends[j - 1]
            k_cache[pg, :, sl_, :] = kr
            v_cache[pg, :, sl_, :] = vr
        kv, q, kps = step_args(s)
        if ev is not None:
            ev[0].record(stream)
        sdi.index_topk(kv, q, kps, k_max, idx_out=idx, workspace=ws_index, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        sdi.attend(kv, q, idx, kps, out=out, workspace=ws_attend, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    def timed_graph(body, reps, count):
        """Capture `count` calls of body(j) into one HIP graph, replay it `reps` times
        back to back between two events; returns (seconds per call, wall seconds)."""
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=cap_stream):
            for j in range(count):
                body(j)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) * 1e-3 / (reps * count), wall

    def index_only(s):
        kv, q, kps = step_args(s)
        sdi.index_topk(kv, q, kps, k_max, idx_out=idx, workspace=ws_index, stream=torch.cuda.current_stream())

    def attend_only(s):
        kv, q, kps = step_args(s)
        sdi.attend(kv, q, idx, kps, out=out, workspace=ws_attend, stream=torch.cuda.current_stream())

    def dense_only(s):
        kv, q, _ = step_args(s)
        sdi.dense(kv, q, out=out, workspace=ws_dense, stream=torch.cuda.current_stream())

    def full_step(s):
        kv, q, kps = step_args(s)
        j = s % n_q
        if growth and j > 0:                              # a0: append this step's token (plain copies)
            pg, sl_, kr, vr = appends[j - 1]
            k_cache[pg, :, sl_, :] = kr
            v_cache[pg, :, sl_, :] = vr
        st = torch.cuda.current_stream()
        sdi.index_topk(kv, q, kps, k_max, idx_out=idx, workspace=ws_index, stream=st)
        sdi.attend(kv, q, idx, kps, out=out, workspace=ws_attend, stream=st)

    for s in range(args.warmup):
        run_step(s)
    torch.cuda.synchronize()
    if args.mode == "graph":
        # steps are replayed from one captured graph of `per` distinct steps (own query each)
        cap_stream = torch.cuda.Stream()
        per = max(d for d in range(1, 17) if args.steps % d == 0 and d <= n_q)
        reps = args.steps // per
        t_step, wall = timed_graph(full_step, reps, per)
        mi, _ = timed_graph(index_only, max(1, reps), per)
        ma, _ = timed_graph(attend_only, max(1, reps), per)
        timing = f"HIP graph replay ({per} distinct steps per graph, {reps} replays)"
        t_step_gpu = t_step
    else:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        t0 = time.perf_counter()
        for s in range(args.steps):
            run_step(args.warmup + s, evs[s])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mi = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3)
        ma = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3)
        t_step_gpu = evs[0][0].elapsed_time(evs[-1][2]) * 1e-3 / args.steps if args.steps > 1 else wall
        timing = "eager launches, events around each call"
    ms_per_step = wall / args.steps * 1e3

    # dense decode of the same layer
    dense_s = None
    if not args.no_dense:
        for s in range(min(args.warmup, 3)):
            dense_only(s)
        torch.cuda.synchronize()
        if args.mode == "graph":
            dense_s, _ = timed_graph(dense_only, max(1, reps // 2), per)
        else:
            dsteps = max(10, args.steps // 2)
            dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(dsteps)]
            for s in range(dsteps):
                dev_ev[s][0].record(stream)
                dense_only(s)
                dev_ev[s][1].record(stream)
            torch.cuda.synchronize()
            dense_s = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_ev]) * 1e-3)

    quest = None
    if args.quest and args.mode == "graph":
        quest = quest_leg(sdi, wl, kv_full, step_args, timed_graph, per, reps, n_q, k_max, idx, out, ws_attend,
                          dense_s)

    labels = None
    if args.labels and args.mode == "graph":
        labels = labels_leg(sdi, wl, kv_full, step_args, timed_graph, per, reps, k_max, idx, out, ws_index,
                            ws_attend, dense_s)

    sampled = None
    if args.sampled and args.mode == "graph":
        sampled = sampled_leg(sdi, wl, kv_full, step_args, timed_graph, per, reps, n_q, k_max, idx, out, ws_index,
                              dense_s)

    cold = {}
    if not args.no_cold and args.mode == "graph":
        # Each launch group right after writing 1 GiB (which flushes the 256 MB Infinity
        # Cache and the L2s), inside HIP graphs: time(flush + group) - time(flush).
        flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        creps = max(1, min(reps, 4))

        def flushed(body):
            def run(s):
                flush.fill_(s & 0xFF)
                if body is not None:
                    body(s)
            return run
        t_flush, _ = timed_graph(flushed(None), creps, per)
        t_fi, _ = timed_graph(flushed(index_only), creps, per)
        t_fa, _ = timed_graph(flushed(attend_only), creps, per)
        t_fs, _ = timed_graph(flushed(full_step), creps, per)
        cold = {"index_us_cold": (t_fi - t_flush) * 1e6, "attend_us_cold": (t_fa - t_flush) * 1e6,
                "step_us_cold": (t_fs - t_flush) * 1e6,
                "cold_timing": "graph replay: each group after a 1 GiB write, minus the write alone"}
        del flush
    if args.calibration_copy_mib > 0:
        src = torch.ones(args.calibration_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # algorithmic bytes per launch, averaged over the distinct steps the graphs replay
    per_steps = per if args.mode == "graph" else 1
    bytes_steps = [algorithmic_bytes((wl.seq_lens + (j if growth else 0)), kps_steps[j if growth else 0].cpu().numpy(),
                                     B, hq, hkv) for j in range(per_steps)]
    b_index, b_attend, b_dense = (float(np.mean([b[i] for b in bytes_steps])) for i in range(3))
    step_bytes = b_index + b_attend
    if cold:
        cold["index_pct_of_peak_cold"] = 100 * b_index / (cold["index_us_cold"] * 1e-6) / PEAK_HBM_BPS
        cold["attend_pct_of_peak_cold"] = 100 * b_attend / (cold["attend_us_cold"] * 1e-6) / PEAK_HBM_BPS
    value = args.steps / wall
    traffic = read_traffic(args.config)
    roofline = {"bound": "hbm", "kernel": "index_topk (score_kernel + select_kernel)",
                "achieved": b_index / mi / 1e9, "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                "frac": b_index / mi / PEAK_HBM_BPS, "traffic": traffic,
                "algorithmic_bytes_per_launch": b_index, "avg_launch_us": mi * 1e6}
    roofline_attend = {"bound": "hbm", "kernel": "attend_kernel",
                       "achieved": b_attend / ma / 1e9, "peak": PEAK_HBM_BPS / 1e9, "unit": "GB/s",
                       "frac": b_attend / ma / PEAK_HBM_BPS, "algorithmic_bytes_per_launch": b_attend,
                       "avg_launch_us": ma * 1e6}
    if cold:
        roofline["frac_cold"] = b_index / (cold["index_us_cold"] * 1e-6) / PEAK_HBM_BPS
        roofline_attend["frac_cold"] = b_attend / (cold["attend_us_cold"] * 1e-6) / PEAK_HBM_BPS
    result = {
        "metric": METRIC, "value": value, "unit": "decode steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": synth.CONFIG_NAMES[args.config] + (f" (ratio {args.ratio})" if args.ratio != 50 else ""),
                   "batch": B, "num_q_heads": hq, "num_kv_heads": hkv, "head_dim": 128, "page_size": 16,
                   "context_max": int(wl.n_max), "k_max": k_max, "sparsity": args.ratio,
                   "layout": wl.meta.get("layout"), "parallelism": "single GPU"},
        "step_GBps": step_bytes / (mi + ma) / 1e9, "step_pct_of_peak": 100 * step_bytes / (mi + ma) / PEAK_HBM_BPS,
        "index_us": mi * 1e6, "attend_us": ma * 1e6, "gpu_step_us": t_step_gpu * 1e6, "timing": timing,
        "roofline": roofline, "roofline_attend": roofline_attend,
    }
    if dense_s is not None:
        result.update({"dense_us": dense_s * 1e6, "dense_steps_per_s": 1.0 / dense_s,
                       "dense_GBps": b_dense / dense_s / 1e9, "dense_pct_of_peak": 100 * b_dense / dense_s / PEAK_HBM_BPS,
                       "speedup_vs_dense": dense_s / (wall / args.steps),
                       "attend_speedup_vs_dense": dense_s / ma})
    if quest is not None:
        result["quest"] = quest
    if labels is not None:
        result["labels"] = labels
    if sampled is not None:
        result["sampled"] = sampled
    result.update(cold)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)      # the host copy is still at step 0
    result["setup_s"] = setup_s
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
