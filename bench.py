#!/usr/bin/env python3
"""Benchmark of the TokenSwift-style hot path on one MI355X.

One step = one pass of the whole path for one LLaMA3.1-8B-shaped layer
(32 query heads, 8 KV heads, head_dim 128, bf16) over one 102,400-token cache:

  1. tree-verify attention of 120 draft queries ([1,3,3,3] tree + 20 four-token
     chains) over the full cache: split-K kernel, then log-sum-exp merge;
  2. partial-KV refresh of the same cache: chunk importance from the 4 latest
     queries -> top-64 of 1600 chunks per KV head -> gather of the 4096-token
     partial cache;
  3. the 4-query draft attention over the partial cache.

The timed step is four kernels: the verify split kernel, which also scores
the chunks on the same reads of K (ts_tree_verify_attn_partials_and_importance);
the merge sharing its grid with the top-k (ts_attn_merge_and_topk); the draft
pass that gathers the chosen chunks as it reads them (ts_kv_gather_and_draft_attn:
split kernel, then its merge). --unfused times the separate launches (split,
merge, importance, top-k, gather, draft split + merge).

Timing (all on the stream every call launches on, torch's current stream):
  * warm-up: at least W steps, then steps until at least --min-warm-s seconds
    have passed and the last three 20-step batches agree within 2% (the chip
    settles at its power limit a few milliseconds into sustained matrix-core
    load), capped at --max-warm-s;
  * the step (value): K steps back to back between two device syncs, wall
    clock, with no event between the steps (an event recorded between two
    launches idles the GPU for several µs); batches of 5 steps with events
    around each give the median/p10/p90;
  * cold steps: each rep first writes a 1 GiB scratch buffer and reads it
    back (outside the events), so that neither the 256 MB last-level cache
    nor the L2 holds any input and no dirty line of the flush is left to be
    written out during the timed call, then times one step;
  * the fused and the unfused step alternated, each timed by events;
  * per-kernel durations: HIP events between the calls of the fused and of
    the unfused step, each settled again first (every event idles the GPU for
    a few µs before the next launch: that gap is inside each call's figure):
    the roofline of the dominant kernel;
  * one ts_tree_verify_attn call (split + merge), cold and warm, at 20,480 and
    102,400 cached tokens (LLaMA3.1-8B) and at 102,400 (LLaMA2-7B MHA).

Inputs are seeded synthetic tensors resident in HBM before timing starts:
the cache and the 4 recent queries of the partial-KV workload (seed 3, 8
chunks per KV head carrying 3x keys) and the drafts of the verify workload
(seed 2: queries, draft K/V, the tree + chains forest). The verify-call lines
run the verify workload with its own cache. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--unfused] [--graph] [--cpu-heads H] [--cpu-seconds S]
                    [--no-cpu-baseline] [--no-verify-lines] [--no-probes] [--calibrate-copy]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per tree-verify step @100K KV (LLaMA3.1-8B layer shape) + % HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
FLUSH_BYTES = 1 << 30           # scratch written before each cold rep


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--min-warm-s", type=float, default=1.0,
                    help="warm up for at least this long (and until step times settle)")
    ap.add_argument("--max-warm-s", type=float, default=8.0)
    ap.add_argument("--cold-reps", type=int, default=30)
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="KV heads of the step the CPU oracle runs for the baseline (of 8)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU baseline repeats its sample until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify-lines", action="store_true",
                    help="skip the per-workload verify-call lines (20K, 100K, MHA 100K)")
    ap.add_argument("--no-probes", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--graph", action="store_true", help="time HIP graph replays of the step instead of eager launches")
    ap.add_argument("--unfused", action="store_true",
                    help="time the step as its separate launches (split, merge, importance, top-k, gather, "
                         "draft split + merge) instead of the four fused kernels")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def to_dev(a, dtype, dev):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def stats(us):
    xs = sorted(us)
    q = lambda p: float(np.percentile(xs, p))
    return {"median": round(q(50), 2), "p10": round(q(10), 2), "p90": round(q(90), 2),
            "mean": round(float(np.mean(xs)), 2), "n": len(xs)}


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


class Timer:
    """Event timing on the current stream, plus the cold-cache flush."""

    def __init__(self, dev):
        import torch
        self.torch = torch
        self.dev = dev
        self.flush_buf = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        self.sink = torch.empty(256, dtype=torch.int32, device=dev)
        self.n_flush = 0

    def events(self, n):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def batches(self, fn, n_batches, per_batch):
        """Per-call µs of `n_batches` batches of `per_batch` back-to-back calls,
        with events only around each batch: an event recorded between two
        launches leaves the GPU idle for several µs before the next one, so
        per-call events would time that idle gap too."""
        ev = self.events(2 * n_batches)
        for b in range(n_batches):
            ev[2 * b].record()
            for _ in range(per_batch):
                fn()
            ev[2 * b + 1].record()
        self.torch.cuda.synchronize()
        return [ev[2 * b].elapsed_time(ev[2 * b + 1]) * 1e3 / per_batch for b in range(n_batches)]

    def back_to_back(self, fn, reps):
        """Per-call µs of `reps` back-to-back calls."""
        ev = self.events(reps + 1)
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        self.torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]

    def flush(self):
        # A 1 GiB write evicts the 256 MB last-level cache and the L2; reading
        # the buffer back then writes those dirty lines out before the timed
        # call starts, so the call competes with no write-back of the flush.
        from long_context_kv_ts_amd import probe
        self.n_flush += 1
        self.flush_buf.fill_(self.n_flush & 0x7FFFFFFF)
        rc = probe.lib().ts_probe_stream_read(self.flush_buf.data_ptr(), FLUSH_BYTES, self.sink.data_ptr(),
                                              self.torch.cuda.current_stream(self.dev).cuda_stream)
        if rc != 0:
            raise RuntimeError(f"flush read failed (hipError {rc})")

    def cold(self, fn, reps):
        """Per-call µs of `reps` calls, each after a 1 GiB scratch write and read-back (outside the events)."""
        ev = self.events(2 * reps)
        for i in range(reps):
            self.flush()
            ev[2 * i].record()
            fn()
            ev[2 * i + 1].record()
        self.torch.cuda.synchronize()
        return [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(reps)]

    def steady(self, fn, min_steps, min_s, max_s, batch=20, tol=0.02):
        """Run `fn` at least `min_steps` times, then in batches until `min_s`
        seconds have passed and the last three batch means agree within `tol`
        (or `max_s` seconds have passed)."""
        for _ in range(min_steps):
            fn()
        self.torch.cuda.synchronize()
        t0 = time.perf_counter()
        means, n = [], min_steps
        while True:
            means.append(float(np.mean(self.back_to_back(fn, batch))))
            n += batch
            el = time.perf_counter() - t0
            last = means[-3:]
            settled = len(last) == 3 and max(last) <= min(last) * (1.0 + tol)
            if (el >= min_s and settled) or el >= max_s:
                return {"steps": n, "seconds": round(el, 2), "settled": settled,
                        "last_batch_means_us": [round(x, 2) for x in last]}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the sharded multi-GPU path is design only, not implemented "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_kv_ts_amd import inputs, ops

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": src.numel() * 2, "bytes_written": dst.numel() * 2}))
        return
    ops.lib()   # fail loudly if the library is missing

    t0 = time.time()
    vc = inputs.workload("llama8b_100k")
    pc = inputs.workload("partial_100k")
    log(f"inputs generated in {time.time() - t0:.1f}s")

    # ---- device-resident inputs and preallocated outputs -------------------
    # one cache for the whole step: the partial-KV workload's
    q = to_dev(vc.q, "bf16", dev)
    kd, vd = to_dev(vc.k_draft, "bf16", dev), to_dev(vc.v_draft, "bf16", dev)
    parent = to_dev(vc.parent, "i32", dev)
    T, Hq, Hkv, D, L = vc.T, vc.Hq, vc.Hkv, vc.D, vc.L
    S = ops.num_splits(T, Hq, Hkv, D, L, torch.bfloat16)
    # the split partials in bf16 (the output is bf16): half the bytes for the merge
    o_part = torch.empty((S, T, Hq, D), dtype=torch.bfloat16, device=dev)
    l_part = torch.empty((S, T, Hq), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)

    pq = to_dev(pc.q, "bf16", dev)
    pk, pv = to_dev(pc.k_cache, "bf16", dev), to_dev(pc.v_cache, "bf16", dev)
    kc, vcache = pk, pv
    pkn, pvn = to_dev(pc.k_new, "bf16", dev), to_dev(pc.v_new, "bf16", dev)
    scores = torch.empty((pc.Hkv, pc.n_chunks), dtype=torch.float32, device=dev)
    idx = torch.empty((pc.Hkv, pc.k), dtype=torch.int32, device=dev)
    idx_s = torch.empty((pc.Hkv, pc.k), dtype=torch.float32, device=dev)
    kp = torch.empty((pc.Hkv, pc.k * pc.chunk, pc.D), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    dout = torch.empty_like(pq)
    dlse = torch.empty((pc.R, pc.Hq), dtype=torch.float32, device=dev)
    dws = ops.alloc_workspace(ops.lib().ts_partial_draft_attn_workspace(
        pc.R, pc.Hq, pc.Hkv, pc.D, pc.k * pc.chunk, ops.TS_BF16, 0), dev)

    def step():
        ops.tree_verify_attn_partials(q, kc, vcache, kd, vd, parent, scale=vc.scale,
                                      o_part=o_part, l_part=l_part)
        ops.attn_merge(o_part, l_part, out=out, lse=lse)
        ops.kv_importance_score(pq, pk, pc.chunk, scale=pc.scale, scores=scores)
        ops.kv_topk_select(scores, pc.k, chunk_idx=idx, chunk_score=idx_s)
        ops.kv_gather(pk, pv, idx, pc.chunk, k_part=kp, v_part=vp)
        ops.partial_draft_attn(pq, kp, vp, pkn, pvn, scale=pc.scale, out=dout, lse=dlse,
                               workspace=dws)

    # The timed step, four kernels: the verify split kernel also scores the
    # cache's chunks on the same reads of K; the merge shares its grid with the
    # top-k; the draft pass gathers the chosen chunks as it reads them, then
    # merges its splits. The per-kernel pass below also runs the separate
    # launches so that each has its own time.
    def step_fused():
        ops.tree_verify_attn_partials_and_importance(q, kc, vcache, kd, vd, parent, pq, pc.chunk, scale=vc.scale,
                                                     imp_scale=pc.scale, o_part=o_part, l_part=l_part,
                                                     scores=scores)
        ops.attn_merge_and_topk(o_part, l_part, scores, pc.k, out=out, lse=lse, chunk_idx=idx, chunk_score=idx_s)
        ops.kv_gather_and_draft_attn(pk, pv, idx, pc.chunk, pq, pkn, pvn, scale=pc.scale, k_part=kp, v_part=vp,
                                     out=dout, lse=dlse, workspace=dws)

    tm = Timer(dev)
    run_step = step if args.unfused else step_fused
    for _ in range(2):
        step()
    # With --graph the step is replayed as one HIP graph (nothing in it
    # allocates or clears memory); by default the launches are eager.
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step()
        timed_step = graph.replay
    else:
        timed_step = run_step
    warm = tm.steady(timed_step, args.warmup, args.min_warm_s, args.max_warm_s)
    log(f"warm-up: {warm}")

    # ---- the step: K steps back to back, wall clock between two syncs --------
    # (no event between the steps: each would leave the GPU idle for a few µs)
    ev = tm.events(2)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        timed_step()
    ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    gpu_us_per_step = ev[0].elapsed_time(ev[1]) * 1e3 / args.steps
    # the spread: batches of 5 steps with events around each batch
    step_warm = stats(tm.batches(timed_step, max(args.steps // 5, 4), 5))
    log(f"step: {ms_per_step * 1e3:.1f} us/step wall, {gpu_us_per_step:.1f} us/step between events; "
        f"5-step batches {step_warm}")

    # ---- cold steps ----------------------------------------------------------
    step_cold = stats(tm.cold(timed_step, args.cold_reps))

    # ---- the fused and the unfused step, alternated --------------------------
    fu, un = [], []
    for _ in range(max(args.steps // 5, 10)):
        fu += tm.batches(step_fused, 1, 5)
        un += tm.batches(step, 1, 5)
    alternated = {"fused": stats(fu), "unfused": stats(un)}

    # ---- per-kernel durations ------------------------------------------------
    # Events between the calls of the step, after settling the instrumented
    # step again (the clock sags for a few dozen launches after the GPU has
    # idled, as between this script's regions). Each recorded event idles the
    # GPU for a few µs before the next launch, and that gap is inside the
    # duration of the call after it; timing each call alone in a loop instead
    # changes the power state (a loop of verify calls alone runs hotter and
    # slower than the step) or times the host's call overhead (the short calls).
    fused_calls = [
        ("verify_split_importance", lambda: ops.tree_verify_attn_partials_and_importance(
            q, kc, vcache, kd, vd, parent, pq, pc.chunk, scale=vc.scale, imp_scale=pc.scale, o_part=o_part,
            l_part=l_part, scores=scores)),
        ("merge_topk", lambda: ops.attn_merge_and_topk(o_part, l_part, scores, pc.k, out=out, lse=lse, chunk_idx=idx,
                                                       chunk_score=idx_s)),
        ("gather_draft_attn", lambda: ops.kv_gather_and_draft_attn(pk, pv, idx, pc.chunk, pq, pkn, pvn, scale=pc.scale,
                                                                   k_part=kp, v_part=vp, out=dout, lse=dlse,
                                                                   workspace=dws)),
    ]
    unfused_calls = [
        ("verify_split", lambda: ops.tree_verify_attn_partials(q, kc, vcache, kd, vd, parent, scale=vc.scale,
                                                               o_part=o_part, l_part=l_part)),
        ("verify_merge", lambda: ops.attn_merge(o_part, l_part, out=out, lse=lse)),
        ("importance", lambda: ops.kv_importance_score(pq, pk, pc.chunk, scale=pc.scale, scores=scores)),
        ("topk", lambda: ops.kv_topk_select(scores, pc.k, chunk_idx=idx, chunk_score=idx_s)),
        ("gather", lambda: ops.kv_gather(pk, pv, idx, pc.chunk, k_part=kp, v_part=vp)),
        ("draft_attn", lambda: ops.partial_draft_attn(pq, kp, vp, pkn, pvn, scale=pc.scale, out=dout, lse=dlse,
                                                      workspace=dws)),
    ]

    def per_call(calls):
        def run(ev):
            for i, (_, fn) in enumerate(calls):
                ev[i].record()
                fn()
            ev[len(calls)].record()
        warm_ev = tm.events(len(calls) + 1)
        tm.steady(lambda: run(warm_ev), 1, 0.5, args.max_warm_s)
        events = [tm.events(len(calls) + 1) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e in events:
            run(e)
        torch.cuda.synchronize()
        per = {n: [e[j].elapsed_time(e[j + 1]) * 1e3 for e in events] for j, (n, _) in enumerate(calls)}
        return ({n: float(np.mean(v)) for n, v in per.items()}, {n: float(np.median(v)) for n, v in per.items()})

    favg, fmed = per_call(fused_calls)
    avg, med = per_call(unfused_calls)

    # ---- roofline of the dominant kernel of the timed step ---------------------
    # the split kernel that also scores the chunks: the verify's QK^T and PV
    # flops plus the importance's QK^T flops (4 queries x 4 heads per KV head)
    flops = verify_flops(vc)
    imp_flops = 2.0 * pc.R * pc.Hq * pc.L * pc.D
    kv_bytes = 2.0 * Hkv * L * D * 2            # K and V of the cache, read once
    dom = "verify_split" if args.unfused else "verify_split_importance"
    t_dom = (avg if args.unfused else favg)[dom] * 1e-6
    dom_flops = flops if args.unfused else flops + imp_flops
    achieved = dom_flops / t_dom / 1e12
    t_split = avg["verify_split"] * 1e-6
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic("attn_split_mfma_kernel<128, 8, 256, 8, false>" if args.unfused
                                            else TRAFFIC_KERNEL),
                "kernel": ("verify split-K (attn_split_mfma_kernel)" if args.unfused else
                           "verify split-K with chunk importance (attn_split_mfma_kernel, importance wave)"),
                "kernel_us": round(t_dom * 1e6, 2),
                "algorithmic_flops": dom_flops, "algorithmic_bytes": kv_bytes,
                "hbm_GBs": round(kv_bytes / t_dom / 1e9, 1),
                "hbm_frac": round(kv_bytes / t_dom / 1e9 / HBM_PEAK_GBS, 4),
                "verify_split_alone": {"us": round(t_split * 1e6, 2),
                                       "TFLOPs": round(flops / t_split / 1e12, 2),
                                       "frac": round(flops / t_split / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}}

    res = {
        "metric": METRIC,
        "value": round(ms_per_step * 1e3, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b layer, one 102400-token bf16 KV cache: tree-verify of 120 drafts "
                               "([1,3,3,3] tree + 20 4-gram chains) + partial-KV refresh of the same cache "
                               "(4 queries, 64 of 1600 64-token chunks) + 4-query draft attention",
                   "T": T, "Hq": Hq, "Hkv": Hkv, "head_dim": D, "kv_len": L, "splits": S,
                   "chunk": pc.chunk, "topk": pc.k},
        "timing": ("graph replay of the step" if graph is not None else "eager launches") +
                  ("" if args.unfused else "; four kernels: verify split with chunk importance, merge with "
                   "top-k, draft split with gather, draft merge") +
                  "; value = wall clock of the back-to-back steps after a settled warm-up, no event between "
                  "steps; step_us.warm = means of 5-step batches; step_us.cold = one step after a 1 GiB "
                  "flush, events around it (one event's idle gap included)",
        "warmup_settled": warm,
        "gpu_us_per_step": round(gpu_us_per_step, 2),
        "step_us": {"warm": step_warm, "cold": step_cold},
        "step_alternated_us": alternated,
        "kernel_us_avg": {n: round(v, 2) for n, v in avg.items()},
        "kernel_us_median": {n: round(v, 2) for n, v in med.items()},
        "step_kernel_us_avg": {n: round(v, 2) for n, v in favg.items()},
        "step_kernel_us_median": {n: round(v, 2) for n, v in fmed.items()},
        "roofline": roofline,
    }

    # ---- one ts_tree_verify_attn call per workload ----------------------------
    if not args.no_verify_lines:
        res["verify_call_us"] = verify_lines(tm, dev, vc, args)
    peaks = None
    if not args.no_probes:
        peaks = measured_peaks(dev)
        res["measured_peaks"] = peaks
        roofline["frac_of_measured_mfma"] = round(achieved / peaks["mfma_bf16"]["sustained_tflops"], 4)

    res["accept_commit_us"] = time_accept_commit(vc, dev, args.steps)
    res["draft_tree_us"] = time_draft_tree(dev, args.steps)
    res["sample_us"] = time_sample(dev, args.steps)
    # the summary page's temperature ablation samples with top-p: temperature 0.8, top-p 0.9, no min-p
    res["sample_top_p_us"] = time_sample(dev, args.steps, temperature=0.8, min_p=0.0, top_p=0.9)
    res["ngram_us"] = time_ngram(dev, args.steps)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(vc, pc, args.cpu_heads, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def verify_flops(c):
    """Algorithmic flops of one verify call: 4*D per (query row, visible key)
    pair, QK^T and PV at 2 flops per multiply-add."""
    vis = 0
    for t in range(c.T):           # |A(t)| summed over draft rows (the ancestor walk of the mask)
        a = t
        while a >= 0:
            vis += 1
            a = int(c.parent[a])
    return 4.0 * c.D * c.Hq * (c.T * c.L + vis)


def verify_lines(tm, dev, vc2, args):
    """One ts_tree_verify_attn call (split + merge, library-chosen splits) per
    workload: median/p10/p90 cold (1 GiB scratch write and read-back before each call,
    events around the call) and warm (means of 5-call back-to-back batches), with %HBM of
    the cache's K+V and %MFMA of 2.5 PF."""
    import torch
    from long_context_kv_ts_amd import inputs, ops
    lines = {}
    for name in ("llama8b_100k", "llama8b_20k", "llama2_mha_100k"):
        t0 = time.time()
        c = vc2 if name == "llama8b_100k" else inputs.workload(name)
        q, kc, vc = to_dev(c.q, "bf16", dev), to_dev(c.k_cache, "bf16", dev), to_dev(c.v_cache, "bf16", dev)
        kd, vd, par = to_dev(c.k_draft, "bf16", dev), to_dev(c.v_draft, "bf16", dev), to_dev(c.parent, "i32", dev)
        log(f"{name}: inputs in {time.time() - t0:.1f}s")
        out = torch.empty_like(q)
        lse = torch.empty((c.T, c.Hq), dtype=torch.float32, device=dev)
        ws = ops.alloc_workspace(ops.verify_workspace_bytes(c.T, c.Hq, c.Hkv, c.D, c.L, torch.bfloat16), dev)
        call = lambda: ops.tree_verify_attn(q, kc, vc, kd, vd, par, scale=c.scale, out=out, lse=lse, workspace=ws)
        tm.steady(call, 3, 0.5, 4.0)
        warm = stats(tm.batches(call, max(args.steps // 5, 4), 5))
        cold = stats(tm.cold(call, args.cold_reps))
        kv = 2.0 * c.Hkv * c.L * c.D * 2
        fl = verify_flops(c)
        t = cold["median"] * 1e-6
        lines[name] = {"cold": cold, "warm": warm, "kv_bytes": kv, "flops": fl,
                       "splits": ops.num_splits(c.T, c.Hq, c.Hkv, c.D, c.L, torch.bfloat16),
                       "hbm_frac_cold": round(kv / t / 1e9 / HBM_PEAK_GBS, 4),
                       "mfma_frac_cold": round(fl / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                       "hbm_frac_warm": round(kv / (warm["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"verify call {name}: cold {cold['median']} us, warm {warm['median']} us")
        del q, kc, vc, kd, vd, par
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return lines


def measured_peaks(dev):
    """What this GPU sustains, from the probe kernels (libts_probe.so)."""
    from long_context_kv_ts_amd import probe
    return probe.measure_all(dev)


def time_accept_commit(vc, dev, reps):
    """Acceptance + KV commit after the step (its own figure, not part of the
    step's value): the verify forest with the target agreeing along one
    4-token tree path, 8 KV heads of bf16 K/V rows committed."""
    import torch
    from long_context_kv_ts_amd import ops
    parent = vc.parent.astype(np.int32)
    T = len(parent)
    draft = (np.arange(T) + 1000).astype(np.int32)
    target = np.full(T + 1, -5, np.int32)
    leaf = max(t for t in range(T) if t < 40 and not (parent == t).any())
    path = []
    a = leaf
    while a >= 0:
        path.append(a)
        a = int(parent[a])
    path = path[::-1]
    target[0] = draft[path[0]]
    for i in range(1, len(path)):
        target[path[i - 1] + 1] = draft[path[i]]
    L = 4096
    kc = torch.zeros((vc.Hkv, L + T, vc.D), dtype=torch.bfloat16, device=dev)
    vcc = torch.zeros_like(kc)
    kd = torch.ones((vc.Hkv, T, vc.D), dtype=torch.bfloat16, device=dev)
    vd = torch.ones_like(kd)
    pt, dt, tt = (torch.from_numpy(x).to(dev) for x in (parent, draft, target))
    n, pth, bonus = ops.accept_commit(pt, dt, tt, 7, kc, vcc, L, kd, vd)
    for _ in range(3):
        ops.accept_commit(pt, dt, tt, 7, kc, vcc, L, kd, vd, n_accepted=n, path=pth, bonus=bonus)
    torch.cuda.synchronize()
    assert int(n.item()) == len(path)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ops.accept_commit(pt, dt, tt, 7, kc, vcc, L, kd, vd, n_accepted=n, path=pth, bonus=bonus)
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / reps, 2)


def time_draft_tree(dev, reps):
    """Candidate tree [1,3,3,3] from 4 positions' fp32 logits over the
    LLaMA3.1 vocabulary of 128,256 tokens (its own figure, not part of value)."""
    import torch
    from long_context_kv_ts_amd import ops
    g = torch.Generator(device=dev)
    g.manual_seed(4)
    logits = torch.randn((4, 128256), device=dev, generator=g)
    ws = ops.alloc_workspace(int(ops.lib().ts_build_draft_tree_workspace(128256, 4)), dev)
    parent, tok, cand = ops.build_draft_tree(logits, [1, 3, 3, 3], workspace=ws)
    for _ in range(3):
        ops.build_draft_tree(logits, [1, 3, 3, 3], parent=parent, draft_tok=tok, cand=cand, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ops.build_draft_tree(logits, [1, 3, 3, 3], parent=parent, draft_tok=tok, cand=cand, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / reps, 2)


def time_sample(dev, reps, temperature=None, min_p=None, top_p=1.0):
    """Target tokens for the 121 verify rows over the LLaMA3.1 vocabulary:
    fp32 logits [121][128256], penalty 1.2 over 1024 tokens, temperature 1,
    min-p 0.1 by default (its own figure, not part of value)."""
    import torch
    from long_context_kv_ts_amd import inputs, ops
    c = inputs.make_sample(dtype="f32")
    logits = torch.from_numpy(c.logits).to(dev)
    hist, parent, dtok = (torch.from_numpy(a).to(dev) for a in (c.hist, c.parent, c.draft_tok))
    u = torch.from_numpy(c.u).to(dev)
    ws = ops.alloc_workspace(int(ops.lib().ts_sample_workspace(c.R, c.V)), dev)
    tok = torch.empty(c.R, dtype=torch.int32, device=dev)
    kw = dict(hist=hist, parent=parent, draft_tok=dtok, window=inputs.PENALTY_WINDOW, penalty=inputs.PENALTY,
              temperature=inputs.TEMPERATURE if temperature is None else temperature,
              min_p=inputs.MIN_P if min_p is None else min_p, top_p=top_p, u=u, tok=tok, workspace=ws)
    for _ in range(3):
        ops.sample_tokens(logits, **kw)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        ops.sample_tokens(logits, **kw)
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / reps, 2)


def time_ngram(dev, reps):
    """One step of the 4-gram table after 102,400 committed tokens: add the
    5 tokens of a verification and retrieve the 20 best 4-grams for a first
    token (its own figure, not part of value)."""
    import torch
    from long_context_kv_ts_amd import inputs, ops
    text = inputs.make_text(102400 + 5 * (reps + 8))
    tokens = torch.from_numpy(text).to(dev)
    table = ops.NgramTable(dev, capacity_log2=18, max_entries=131072)
    table.update(tokens, 0, 102400)
    first = torch.zeros(1, dtype=torch.int32, device=dev)            # the most frequent token id
    ws = ops.alloc_workspace(int(ops.lib().ts_ngram_retrieve_workspace(table.max_entries, 20)), dev)
    out = (torch.empty((20, 4), dtype=torch.int32, device=dev), torch.empty(20, dtype=torch.int32, device=dev),
           torch.empty(1, dtype=torch.int32, device=dev))
    n = 102400
    for _ in range(3):
        table.update(tokens, n, n + 5)
        table.retrieve(first, 20, out_tok=out[0], out_count=out[1], n_found=out[2], workspace=ws)
        n += 5
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        table.update(tokens, n, n + 5)
        table.retrieve(first, 20, out_tok=out[0], out_count=out[1], n_found=out[2], workspace=ws)
        n += 5
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / reps, 2)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_split_importance_102400_hbm_traffic.txt")
TRAFFIC_KERNEL = "attn_split_mfma_kernel<128, 8, 256, 8, true>"
KERNEL_SOURCES = [os.path.join(ROOT, "long_context_kv_ts_amd", "csrc", f) for f in ("attn_mfma.hip", "common.h")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs, scaled by what the same counters read for a plain copy of
    known size; None if the counters are of another kernel or its source has
    changed since."""
    try:
        kv = dict(line.split("=", 1) for line in open(TRAFFIC_FILE) if "=" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel") != kernel or kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return round(float(kv["fetch_kib"]) * float(kv["fetch_scale"]) * 1024
                     + float(kv["write_kib"]) * float(kv["write_scale"]) * 1024)
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(vc, pc, heads, min_seconds):
    """The oracle on `heads` of the 8 KV heads of one step, repeated until
    `min_seconds` have passed (at least once); the mean is scaled to the step."""
    import oracle
    try:
        import threadpoolctl
        blas = threadpoolctl.threadpool_info()
        threads = max([b.get("num_threads", 1) for b in blas] or [1])
    except Exception:
        threads = None
    cores = len(os.sched_getaffinity(0))
    hs = list(range(heads))
    G = pc.Hq // pc.Hkv
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.verify_attn_ref(vc.q, pc.k_cache, pc.v_cache, vc.k_draft, vc.v_draft, vc.parent,
                               vc.scale, "bf16", heads=hs)
        s = oracle.importance_ref(pc.q, pc.k_cache, pc.scale, pc.chunk, "bf16", heads=hs)
        idx, _ = oracle.topk_ref(s[hs], pc.k)
        kp, vp = oracle.gather_ref(pc.k_cache[hs], pc.v_cache[hs], idx, pc.chunk)
        oracle.draft_attn_ref(pc.q[:, :heads * G], kp, vp, pc.k_new[hs], pc.v_new[hs], pc.scale, "bf16")
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    scale = vc.Hkv / heads
    what = "the whole step" if heads == vc.Hkv else f"{heads} of {vc.Hkv} KV heads of one step"
    return {"value": round(dt / reps * 1e6 * scale, 1), "unit": "us", "cores": threads or cores,
            "host_cores": cores, "kind": "oracle",
            "sample": f"{what} (verify + importance + top-k + gather + draft attention), float64 numpy, "
                      f"mean of {reps} runs over {dt:.1f} s" + (f", time x{scale:g}" if heads != vc.Hkv else "")}


if __name__ == "__main__":
    main()
