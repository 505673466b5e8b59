#!/usr/bin/env python3
"""Paged MLA decode benchmark on one MI355X.

One step = one decode call over one batch (mla_decode_paged's two kernels: the
split-KV decode, mla_decode_splitkv, and the log-sum-exp combine,
mla_combine_splits), with q, the paged cache and the split-KV schedule already
resident in HBM.  The schedule (mla_get_metadata) is computed once per decode
step and shared by every layer's decode call in the FlashMLA usage ("OpenSourceWeek
Day 1 -- Demystifying DeepSeek's FlashMLA", §V.2), so it is timed on its own and
reported beside the step (schedule_ms, ms_per_step_with_schedule).  The timed
steps are captured, in order, into HIP graphs of up to 25 consecutive steps each
and every graph is replayed once (a graph launch costs the GPU ~5 us, which one
graph per step would add to every step).  Step i reads cache copy i mod C, with
enough copies C that the working set exceeds twice the 256 MB MALL, so reads
come from HBM.

The headline workload (--config, default spec_decode_causal, the largest) gives
the line's value; every other workload is timed in the same run and listed under
"workloads" with the same fields.  Prints ONE JSON line:
  value          algorithmic bytes per step / wall time per step (TB/s)
  tflops         algorithmic flops per step / wall time per step
  roofline       the decode kernel against MI355X's published peak (HBM or
                 bf16 MFMA, whichever bounds the workload), from HIP events
                 around graphs of back-to-back launches of the kernel
  step_percentiles_ms  p10 / median / p90 of >= 100 eager steps
  copy_bandwidth a plain device copy's rate on this GPU (context)
  cpu_baseline   the fp64 CPU oracle on the host cores over a bounded sample
                 of the headline workload (a reported baseline)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config {0..4}] [--only]
                       [--kv {bf16,fp8}] [--op {decode,absorb,append,sparse}]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
MALL_BYTES = 256 << 20
STEPS_PER_GRAPH = 25


def algorithmic(w, row_bytes=576 * 2):
    """Bytes and flops the method must move / compute for one step.

    bytes: every valid latent+rope row once (V is reused from the same bytes),
    the queries in, out + lse out, block-table entries and lengths.
    flops: 2 * keys * (576 + 512) per query row (scores and P.V)."""
    import numpy as np
    L = w.cache_seqlens.astype(np.int64)
    nb = (L + 63) // 64
    kv = int(L.sum()) * w.h_kv * row_bytes
    qio = w.batch * w.s_q * w.h_q * (576 * 2 + 512 * 2 + 4)
    meta = int(nb.sum()) * 4 + w.batch * 4
    if w.causal:
        keys = sum(int(max(0, Li - w.s_q + s + 1)) for Li in L for s in range(w.s_q)) * w.h_q
    else:
        keys = int(L.sum()) * w.s_q * w.h_q
    flops = 2 * keys * (576 + 512)
    return kv + qio + meta, flops, kv


def source_digest():
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_wide.hip", "decode_qkpv.hip", "decode_common.h", "mla_kernels.h"):
        with open(os.path.join(ROOT, "paged_mla_decode_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload, launch_kind):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary
    (profiles/decode_hbm_traffic.md), or None when missing or taken on a
    different version of the kernel."""
    path = os.path.join(ROOT, "profiles", "decode_hbm_traffic.md")
    try:
        with open(path) as fh:
            lines = fh.read().splitlines()
    except OSError:
        return None
    digest = source_digest()
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[0] == workload and cells[2] == launch_kind:
            if cells[1] != digest:
                return None
            try:
                return int(float(cells[5]))
            except ValueError:
                return None
    return None


def cpu_baseline(w, target_s, row_bytes=576 * 2):
    """The oracle as it stands, on the host cores, over a bounded sample of the
    workload: whole passes repeated for about target_s seconds when a pass is
    shorter than that, else the first n sequences (all their query rows) with n
    chosen from a one-sequence probe so that the run takes about target_s."""
    import numpy as np

    import oracle
    orc = oracle.default()
    cores = len(os.sched_getaffinity(0))
    orc.set_threads(cores)
    per_seq = w.s_q * w.h_q

    def sample_bytes_flops(n):
        sub = workloads_subset(w, n)
        by, fl, _ = algorithmic(sub, row_bytes)
        return by, fl

    t0 = time.perf_counter()
    orc.decode(w, sel=np.arange(per_seq, dtype=np.int64))
    probe = max(time.perf_counter() - t0, 1e-6)
    if probe * w.batch <= target_s:
        runs = 0
        t0 = time.perf_counter()
        while True:
            orc.decode(w)
            runs += 1
            el = time.perf_counter() - t0
            if el >= target_s or runs >= 1000:
                break
        n, per_run = w.batch, el / runs
        what = f"the whole workload ({w.batch} sequences, {w.batch * per_seq} query rows), fp64, " \
               f"repeated {runs}x over {el:.1f} s; {per_run * 1e3:.1f} ms per pass"
    else:
        n = int(min(w.batch, max(1, target_s / probe)))
        for _ in range(2):  # a second, larger sample when the probe overestimated
            t0 = time.perf_counter()
            orc.decode(w, sel=np.arange(n * per_seq, dtype=np.int64))
            per_run = time.perf_counter() - t0
            if per_run >= 0.5 * target_s or n >= w.batch:
                break
            n = int(min(w.batch, n * target_s / per_run))
        what = f"the first {n} of {w.batch} sequences ({n * per_seq} query rows, " \
               f"{int(w.cache_seqlens[:n].sum())} cached tokens), fp64, one pass of {per_run:.1f} s"
    by, fl = sample_bytes_flops(n)
    return {"value": round(by / per_run / 1e12, 6), "unit": "TB/s", "cores": orc.num_threads(), "kind": "oracle",
            "tflops": round(fl / per_run / 1e12, 6), "sample": what}


def workloads_subset(w, n):
    """The first n sequences of workload w (same cache and tables), for sizing
    the CPU baseline's sample."""
    import dataclasses
    return dataclasses.replace(w, batch=n, cache_seqlens=w.cache_seqlens[:n], block_table=w.block_table[:n],
                               q=w.q[:n])


def timed_steps(torch, step, K, W, eager=False):
    """Wall time (ms) per step of exactly K steps step(0) .. step(K-1), between
    synchronize() calls, after W untimed warm-up steps.  The K steps are captured,
    in order, into HIP graphs of up to STEPS_PER_GRAPH steps, each replayed once
    (and once more untimed beforehand).  Returns (ms, launch mode, steps per graph)."""
    graphs = None
    per_graph = max(1, min(K, STEPS_PER_GRAPH))
    if not eager:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            graphs = []
            with torch.cuda.stream(s):
                for g0 in range(0, K, per_graph):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        for i in range(g0, min(g0 + per_graph, K)):
                            step(i)
                    graphs.append(g)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
        except Exception as e:  # graphs unavailable: time eager launches
            print(f"graph capture failed ({e}); timing eager launches", file=sys.stderr)
            graphs = None
    for i in range(W):
        step(i)
    for g in graphs or []:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs is not None:
        for g in graphs:
            g.replay()
    else:
        for i in range(K):
            step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / K
    return ms, ("hip_graph" if graphs is not None else "eager"), (per_graph if graphs is not None else None)


def graph_kernel_ms(torch, launches, per_graph=25, n_graphs=4):
    """Average duration (ms) of the kernel each `launches[k](i)` enqueues.

    The i = 0 .. per_graph*n_graphs-1 launches of a kernel are captured into
    n_graphs graphs of per_graph back-to-back launches; every replay is
    bracketed by HIP events on the launch stream (torch's current stream), after
    one untimed replay of the same kernel, and a launch's duration is the
    bracketed time / per_graph (the in-graph dispatch of the next launch
    included).  Returns [(mean, [mean of each graph])] per kernel."""
    import numpy as np
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(s):
        for fn in launches:
            gs = []
            for j in range(n_graphs):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    for i in range(per_graph):
                        fn(j * per_graph + i)
                gs.append(g)
            graphs.append(gs)
    torch.cuda.current_stream().wait_stream(s)
    for gs in graphs:
        for g in gs:
            g.replay()
    torch.cuda.synchronize()
    res = []
    for gs in graphs:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in gs]
        gs[0].replay()  # the kernel running at its steady clock before the first bracket
        for g, e in zip(gs, ev):
            e[0].record()
            g.replay()
            e[1].record()
        torch.cuda.synchronize()
        per = [e[0].elapsed_time(e[1]) / per_graph for e in ev]
        res.append((float(np.mean(per)), [round(x, 5) for x in per]))
    return res


def bench_absorb(args, torch, mla, workloads, dev):
    """Time mla_absorb_q and mla_unabsorb_out for the workload's b*s_q tokens and
    h_q heads: K steps (absorb + unabsorb) replayed from graphs, per-kernel times
    from HIP events around graphs of back-to-back launches."""
    import numpy as np
    cfg = workloads.CONFIGS[args.config]
    b, s_q, h = cfg["batch"], cfg["s_q"], cfg["h_q"]
    T = b * s_q
    lay = workloads.make_layer_inputs(b, s_q, h, seed=args.config)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    qn, qr, wuk, wuv = up(lay.q_nope), up(lay.q_rope), up(lay.w_uk), up(lay.w_uv)
    q_abs = torch.empty((b, s_q, h, 576), dtype=torch.bfloat16, device=dev)
    o_lat = torch.randn((b, s_q, h, 512), device=dev).to(torch.bfloat16)
    out = torch.empty((b, s_q, h, 128), dtype=torch.bfloat16, device=dev)
    # algorithmic bytes / flops of each GEMM: weights once, activations in and out
    by_abs = 2 * (h * 128 * 512 + T * h * (128 + 64 + 576))
    by_un = 2 * (h * 128 * 512 + T * h * (512 + 128))
    fl = 2 * T * h * 128 * 512

    def absorb(i):
        mla.mla_absorb_q(qn, qr, wuk, out=q_abs)

    def unabsorb(i):
        mla.mla_unabsorb_out(o_lat, wuv, out=out)

    for i in range(3):
        absorb(i)
        unabsorb(i)
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    ms, _, _ = timed_steps(torch, lambda i: (absorb(i), unabsorb(i)), K, W)
    (da, _), (du, _) = graph_kernel_ms(torch, [absorb, unabsorb])
    d = [da, du]
    n_ev = 100
    gbs = [by_abs / (d[0] * 1e-3) / 1e9, by_un / (d[1] * 1e-3) / 1e9]
    line = {
        "metric": "MLA absorption GEMMs bf16 (q~ = W_UK^T q_nope, out = W_UV o_lat): achieved TB/s",
        "value": round((by_abs + by_un) / (ms * 1e-3) / 1e12, 4), "unit": "TB/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg["name"], "tokens": T, "h_q": h, "d_nope": 128, "d_latent": 512, "d_v": 128},
        "algorithmic": {"absorb_bytes": by_abs, "unabsorb_bytes": by_un, "flops_each": fl},
        "kernel_ms": {"absorb": round(float(d[0]), 5), "unabsorb": round(float(d[1]), 5), "launches": n_ev},
        "roofline": {"bound": "hbm", "achieved": round(gbs[0], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs[0] / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "absorb_q",
                     "unabsorb_achieved": round(gbs[1], 1), "unabsorb_frac": round(gbs[1] / HBM_PEAK_GBS, 4)},
    }
    print(json.dumps(line))


def bench_append(args, torch, mla, workloads, dev):
    """Time mla_kv_append for one decode step of the workload: every sequence
    appends s_q new cache rows after its current length (steps replayed from
    graphs; the kernel time from HIP events around graphs of back-to-back launches)."""
    import numpy as np
    cfg = workloads.CONFIGS[args.config]
    w0 = workloads.config_workload(args.config)
    s_new = args.append_tokens or cfg["s_q"]
    w, before, new_kv = workloads.make_append_case(w0.cache_seqlens, s_new, h_q=w0.h_q, seed=args.config)
    del w0
    kc = torch.from_numpy(w.kcache.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(before).to(dev)
    nk = torch.from_numpy(new_kv.view(np.int16)).to(dev).view(torch.bfloat16)
    nl = torch.empty_like(sl)
    rows = w.batch * s_new * w.h_kv
    by = 2 * rows * 576 * 2 + 4 * w.batch * 2 + 4 * w.batch * ((s_new + 63) // 64 + 1)

    def step(i):
        mla.mla_kv_append(nk, sl, bt, kc, new_seqlens=nl)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    ms, _, _ = timed_steps(torch, step, K, W)
    (d, _), = graph_kernel_ms(torch, [step])
    n_ev = 100
    gbs = by / (d * 1e-3) / 1e9
    line = {
        "metric": "paged KV append bf16 (new latent+rope rows scattered into 64-token pages): achieved TB/s",
        "value": round(by / (ms * 1e-3) / 1e12, 4), "unit": "TB/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": w.batch, "s_new": s_new, "h_kv": w.h_kv, "rows": rows},
        "algorithmic": {"bytes_per_step": by},
        "kernel_ms": {"append": round(d, 5), "launches": n_ev},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "kv_append"},
    }
    print(json.dumps(line))


def bench_sparse(args, torch, mla, workloads, dev):
    """Token-sparse decode: 64 sequences of U[4096, 16384] tokens, --sparse-heads
    query heads (128 by default; 16 is one GPU's eighth of a 128-head model),
    each query attending to a top-2048 selection (uniform distinct positions).  A step is the decode of the kept rows (decode + combine),
    replayed from graphs of consecutive steps; the preparation (list -> row offsets) and the schedule run
    once per step in use and are timed on their own."""
    import numpy as np
    rng = np.random.default_rng(20)
    lens = rng.integers(4096, 16385, size=64)
    w = workloads.make_workload(lens, s_q=1, h_q=args.sparse_heads, seed=20, name="sparse_topk2048")
    idx, ptr = workloads.make_sparse_indices(w, args.topk, seed=20)
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kc_host = torch.from_numpy(w.kcache.view(np.int16))
    ncopies = max(1, math.ceil(2 * MALL_BYTES / w.kcache.nbytes))
    kcs = [kc_host.to(dev).view(torch.bfloat16) for _ in range(ncopies)]
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    ti = torch.from_numpy(idx).to(dev)
    tp = torch.from_numpy(ptr).to(dev)
    offs, counts = mla.mla_sparse_prepare(ti, tp, 1, bt, sl, w.num_pages, 1)
    rows = w.h_q
    P, ws_bytes = mla.mla_plan(w.batch, rows, 1)
    md, ns = mla.mla_get_metadata(counts, rows, 1, num_parts=P)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, 1, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, 1, w.h_q), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    kept = int(counts.sum().item())
    by = kept * 576 * 2 + w.batch * w.h_q * (576 * 2 + 512 * 2 + 4) + kept * 4
    fl = 2 * kept * w.h_q * (576 + 512)

    def step(c):
        mla.mla_sparse_decode(q, kcs[c], offs, tp, counts, 512, md, ns, w.scale, out, lse, ws, nnz=ti.shape[0])

    for c in range(min(3, ncopies)):
        step(c)
    torch.cuda.synchronize()
    K, W = args.steps, args.warmup
    ms, _, _ = timed_steps(torch, lambda i: step(i % ncopies), K, W)
    (t_step, _), (t_prep, _), (t_md, _) = graph_kernel_ms(torch, [
        lambda i: step(i % ncopies),
        lambda i: mla.mla_sparse_prepare(ti, tp, 1, bt, sl, w.num_pages, 1, offsets=offs, counts=counts),
        lambda i: mla.mla_get_metadata(counts, rows, 1, num_parts=P, out=(md, ns))])
    n_ev = 100
    tf = fl / (t_step * 1e-3) / 1e12
    gbs = by / (t_step * 1e-3) / 1e9
    bound = "hbm" if fl / by < RIDGE else "mfma"
    roof = ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(gbs / HBM_PEAK_GBS, 4)} if bound == "hbm" else
            {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(tf / BF16_PEAK_TFLOPS, 4)})
    roof.update({"traffic": None, "kernel": "sparse decode + combine (mla_sparse_decode)"})
    line = {
        "metric": "token-sparse MLA decode bf16 (top-k rows per query): achieved TB/s & TFLOPS",
        "value": round(by / (ms * 1e-3) / 1e12, 4), "unit": "TB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "sparse_topk", "batch": w.batch, "s_q": 1, "h_q": w.h_q, "h_kv": 1,
                   "topk": args.topk, "seqlens": "uniform [4096, 16384], seed 20", "kept_rows": kept,
                   "num_parts": P, "cache_copies": ncopies},
        "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
        "algorithmic": {"bytes_per_step": by, "flops_per_step": fl},
        "kernel_ms": {"decode_step": round(t_step, 5), "prepare": round(t_prep, 5), "metadata": round(t_md, 5),
                      "launches": n_ev},
        "roofline": roof,
    }
    print(json.dumps(line))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3,
                    help="headline workload index 0..4 (default 3: spec_decode_causal, the largest)")
    ap.add_argument("--only", action="store_true",
                    help="time the headline workload only (by default every workload is timed and listed "
                         "under 'workloads')")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python instead of graphs")
    ap.add_argument("--kv", choices=["bf16", "fp8"], default="bf16",
                    help="cache format of the decode step (fp8: the 656-byte FP8 rows)")
    ap.add_argument("--append-tokens", type=int, default=0,
                    help="--op append: rows appended per sequence (default: the workload's s_q)")
    ap.add_argument("--topk", type=int, default=2048, help="--op sparse: entries selected per query")
    ap.add_argument("--sparse-heads", type=int, default=128, help="--op sparse: query heads (one KV head)")
    ap.add_argument("--op", choices=["decode", "absorb", "append", "sparse"], default="decode",
                    help="decode (default): the decode step; absorb: the two absorption GEMMs of the "
                         "workload's query tokens and heads (one JSON line of their own)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(no collectives or sharding); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_mla_decode_02_amd as mla
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            b_.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": args.steps}))
        return
    if args.op == "absorb":
        bench_absorb(args, torch, mla, workloads, dev)
        return
    if args.op == "append":
        bench_append(args, torch, mla, workloads, dev)
        return
    if args.op == "sparse":
        bench_sparse(args, torch, mla, workloads, dev)
        return
    fp8 = args.kv == "fp8"
    K, W = args.steps, args.warmup
    headline = measure_decode(args.config, K, W, torch, mla, workloads, dev, fp8, eager=args.eager)
    others = []
    if not args.only:
        for idx in sorted(workloads.CONFIGS):
            if idx != args.config:
                others.append(measure_decode(idx, max(K, 100), W, torch, mla, workloads, dev, fp8))
                torch.cuda.empty_cache()
    copy = copy_bandwidth(torch, dev)

    h = headline
    line = {
        "metric": ("paged MLA decode, FP8 latent cache (bf16 compute): achieved TB/s & TFLOPS, % of MI355X "
                   "roofline") if fp8 else "paged MLA decode bf16: achieved TB/s & TFLOPS, % of MI355X roofline",
        "value": h["step_tbps"],
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": h["step_ms"],
        "schedule_ms": h["kernel_ms"]["metadata"],
        "ms_per_step_with_schedule": round(h["step_ms"] + h["kernel_ms"]["metadata"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": h["config"],
        "tflops": h["step_tflops"],
        "roofline_frac_step": h["roofline_frac_step"],
        "algorithmic": h["algorithmic"],
        "kernel_ms": h["kernel_ms"],
        "step_percentiles_ms": h["step_percentiles_ms"],
        "roofline": h["roofline"],
        "copy_bandwidth": copy,
        "workloads": [summary(h)] + [summary(o) for o in others],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(h["workload"], args.cpu_seconds,
                                            mla.FP8_ROW_BYTES if fp8 else 576 * 2)
    print(json.dumps(line))


def summary(r):
    """The per-workload entry of the JSON line (everything but the inputs)."""
    keys = ("config", "step_ms", "step_tbps", "step_tflops", "roofline_frac_step", "kernel_ms",
            "step_percentiles_ms", "roofline", "decode_hbm_frac", "decode_mfma_frac")
    out = {k: r[k] for k in keys}
    out["workload"] = r["config"]["workload"]
    return out


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=20):
    """A plain device-to-device copy of nbytes (torch copy_), events around reps
    back-to-back copies: the streaming rate the chip reaches on this machine, as
    context for the kernels' HBM fractions (read + write bytes per second)."""
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    gbs = 2 * nbytes / (ms * 1e-3) / 1e9
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": round(ms, 4), "GBs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "kind": "torch copy_ (device to device)"}


def eager_percentiles(torch, fn, n):
    """p10 / median / p90 (ms) of n eager launches of fn(i), each bracketed by
    HIP events on the launch stream; a GPU spin first lets the host enqueue all
    of them, so the launches run back to back (each bracket includes the
    dispatch of its first kernel)."""
    import numpy as np
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(60e6))
    for i in range(n):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    d = np.array([s.elapsed_time(e) for s, e in ev])
    return {"p10": round(float(np.percentile(d, 10)), 5), "median": round(float(np.median(d)), 5),
            "p90": round(float(np.percentile(d, 90)), 5), "launches": n,
            "timing": "HIP events around each eager step (decode + combine), queue pre-filled"}


def measure_decode(idx, K, W, torch, mla, workloads, dev, fp8, eager=False):
    """Time one workload's decode step (decode + combine) and its kernels."""
    import numpy as np
    cfg = workloads.CONFIGS[idx]
    w = workloads.config_workload(idx)
    row_bytes = mla.FP8_ROW_BYTES if fp8 else 576 * 2
    bytes_step, flops_step, kv_bytes = algorithmic(w, row_bytes)

    # inputs resident in HBM; enough cache copies that the rotation exceeds twice
    # the MALL (at most 32 copies: the tiny workload stays cache-resident)
    if fp8:
        kc_host = torch.from_numpy(workloads.make_fp8_cache(w, seed=idx))
    else:
        kc_host = torch.from_numpy(w.kcache.view(np.int16))
    kc_bytes = kc_host.numel() * kc_host.element_size()
    ncopies = min(32, max(1, math.ceil(2 * MALL_BYTES / kc_bytes)))
    mall_defeated = ncopies * kc_bytes >= 2 * MALL_BYTES
    kcs = [kc_host.to(dev) if fp8 else kc_host.to(dev).view(torch.bfloat16) for _ in range(ncopies)]
    del kc_host
    decode_fn = mla.mla_decode_splitkv_fp8 if fp8 else mla.mla_decode_splitkv
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    P, ws_bytes = mla.mla_plan(w.batch, w.rows, w.h_kv)
    md = torch.empty((P, 8), dtype=torch.int32, device=dev)
    ns = torch.empty((w.batch + 1,), dtype=torch.int32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((w.batch, w.s_q, w.h_q, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=dev)

    def schedule():
        mla.mla_get_metadata(sl, w.rows, w.h_kv, num_parts=P, out=(md, ns))

    def decode_one(c):
        decode_fn(q, kcs[c], bt, sl, w.dv, md, ns, w.causal, w.scale, out, lse, ws)

    def combine_one(c):
        mla.mla_combine_splits(q, kcs[c], bt, sl, w.dv, md, ns, w.causal, w.scale, out, lse, ws)

    def step(c):
        decode_one(c)
        combine_one(c)

    schedule()
    for i in range(3):
        step(i % ncopies)  # eager warm-up (kernel attributes, allocator)
    torch.cuda.synchronize()
    # the rows of split sequences get out / lse from the combine, the others from the decode
    chunks = np.diff(ns.cpu().numpy().astype(np.int64))
    per_seq_out = w.s_q * w.h_q * (512 * 2 + 4)
    combine_out_bytes = int(np.count_nonzero(chunks > 1)) * per_seq_out
    decode_bytes = bytes_step - combine_out_bytes

    # timed region: exactly K steps of decode + combine, replayed from graphs
    ms_per_step, mode, per_graph = timed_steps(torch, lambda i: step(i % ncopies), K, W, eager=eager)
    if mode == "hip_graph":
        (dec_ms, dec_g), (comb_ms, _), (meta_ms, _) = graph_kernel_ms(
            torch, [lambda i: decode_one(i % ncopies), lambda i: combine_one(i % ncopies), lambda i: schedule()])
        timing = "HIP events around graph replays of 25 back-to-back launches of the kernel, 4 graphs"
    else:
        dec_g = None
        dec_ms = eager_percentiles(torch, lambda i: decode_one(i % ncopies), 100)["median"]
        comb_ms = eager_percentiles(torch, lambda i: combine_one(i % ncopies), 100)["median"]
        meta_ms = eager_percentiles(torch, lambda i: schedule(), 100)["median"]
        timing = "median of HIP events around 100 eager launches of the kernel"
    pct = eager_percentiles(torch, lambda i: step(i % ncopies), max(100, K))

    intensity = flops_step / bytes_step
    bound = "hbm" if intensity < RIDGE else "mfma"
    dec_gbs = decode_bytes / (dec_ms * 1e-3) / 1e9
    dec_tflops = flops_step / (dec_ms * 1e-3) / 1e12
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dec_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(dec_tflops, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dec_tflops / BF16_PEAK_TFLOPS, 4)}
    roof["traffic"] = traffic_from_profiles(cfg["name"], "decode_fp8" if fp8 else "decode")
    roof["kernel"] = "decode (mla_decode_splitkv_fp8)" if fp8 else "decode (mla_decode_splitkv)"
    roof["launch_ms"] = round(float(dec_ms), 5)
    roof["algorithmic_per_launch"] = ({"bytes": int(decode_bytes)} if bound == "hbm" else {"flops": int(flops_step)})

    res = {
        "workload": w,
        "config": {
            "workload": cfg["name"], "batch": w.batch, "s_q": w.s_q, "h_q": w.h_q, "h_kv": w.h_kv,
            "d_qk": 576, "dv": 512, "page_block_size": 64, "causal": w.causal,
            "seqlens": {"kind": cfg["lens"][0], "params": list(cfg["lens"][1:]), "seed": w.seed,
                        "total_tokens": int(w.cache_seqlens.sum())},
            "softmax_scale": w.scale, "num_parts": P, "cache_copies": ncopies, "mall_defeated": mall_defeated,
            "launch": mode, "steps_per_graph": per_graph,
            "kv_format": "fp8_e4m3 rows of 656 B (4 power-of-two scales, bf16 rope)" if fp8 else "bf16",
        },
        "step_ms": round(ms_per_step, 5),
        "step_tbps": round(bytes_step / (ms_per_step * 1e-3) / 1e12, 4),
        "step_tflops": round(flops_step / (ms_per_step * 1e-3) / 1e12, 3),
        "roofline_frac_step": round(max(bytes_step / (HBM_PEAK_GBS * 1e9), flops_step / (BF16_PEAK_TFLOPS * 1e12))
                                    / (ms_per_step * 1e-3), 4),
        "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "decode_mfma_frac": round(dec_tflops / BF16_PEAK_TFLOPS, 4),
        "algorithmic": {"bytes_per_step": int(bytes_step), "flops_per_step": int(flops_step),
                        "flop_per_byte": round(intensity, 2), "decode_bytes": int(decode_bytes),
                        "combine_out_bytes": int(combine_out_bytes)},
        "kernel_ms": {"metadata": round(float(meta_ms), 5), "decode": round(float(dec_ms), 5),
                      "combine": round(float(comb_ms), 5), "decode_per_graph": dec_g, "timing": timing},
        "step_percentiles_ms": pct,
        "roofline": roof,
    }
    del kcs, q, bt, sl, md, ns, ws, out, lse
    return res


if __name__ == "__main__":
    main()
