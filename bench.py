#!/usr/bin/env python3
"""Benchmark of the TokenSwift-style hot path on one MI355X.

One step = one pass of the whole path for one LLaMA3.1-8B-shaped layer
(32 query heads, 8 KV heads, head_dim 128, bf16) over a 102,400-token cache:

  1. tree-verify attention of 120 draft queries ([1,3,3,3] tree + 20 four-token
     chains) over the full cache: split-K kernel, then log-sum-exp merge;
  2. partial-KV refresh: chunk importance from the 4 latest queries ->
     top-64 of 1600 chunks per KV head -> gather of the 4096-token partial cache;
  3. the 4-query draft attention over the partial cache.

The verify merge and the chunk importance depend on nothing of each other and
run as one launch (ts_attn_merge_and_importance; --unfused keeps two). The
per-kernel times come from a second pass with the two apart and HIP events
between kernels.

Inputs are seeded synthetic tensors resident in HBM before timing starts
(verify inputs: seed 2; partial-KV inputs: seed 3, with 8 chunks per KV head
carrying 3x keys). Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--unfused] [--graph] [--cpu-heads H] [--cpu-seconds S]
                    [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per tree-verify step @100K KV (LLaMA3.1-8B layer shape) + % HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="KV heads of the step the CPU oracle runs for the baseline (of 8)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU baseline repeats its sample until this much time has passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="time HIP graph replays of the step instead of eager launches")
    ap.add_argument("--unfused", action="store_true",
                    help="time the merge and the importance as two launches (default: one launch, "
                         "ts_attn_merge_and_importance)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


def to_dev(a, dtype, dev):
    import torch
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    print(f"# inputs generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # ---- device-resident inputs and preallocated outputs -------------------
    q = to_dev(vc.q, "bf16", dev)
    kc, vcache = to_dev(vc.k_cache, "bf16", dev), to_dev(vc.v_cache, "bf16", dev)
    kd, vd = to_dev(vc.k_draft, "bf16", dev), to_dev(vc.v_draft, "bf16", dev)
    parent = to_dev(vc.parent, "i32", dev)
    T, Hq, Hkv, D, L = vc.T, vc.Hq, vc.Hkv, vc.D, vc.L
    S = ops.num_splits(T, Hq, Hkv, D, L, torch.bfloat16)
    o_part = torch.empty((S, T, Hq, D), dtype=torch.float32, device=dev)
    l_part = torch.empty((S, T, Hq), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)

    pq = to_dev(pc.q, "bf16", dev)
    pk, pv = to_dev(pc.k_cache, "bf16", dev), to_dev(pc.v_cache, "bf16", dev)
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

    names = ["verify_split", "verify_merge", "importance", "topk", "gather", "draft_attn"]

    def step(ev=None):
        rec = (lambda i: ev[i].record()) if ev is not None else (lambda i: None)
        rec(0)
        ops.tree_verify_attn_partials(q, kc, vcache, kd, vd, parent, scale=vc.scale,
                                      o_part=o_part, l_part=l_part)
        rec(1)
        ops.attn_merge(o_part, l_part, out=out, lse=lse)
        rec(2)
        ops.kv_importance_score(pq, pk, pc.chunk, scale=pc.scale, scores=scores)
        rec(3)
        ops.kv_topk_select(scores, pc.k, chunk_idx=idx, chunk_score=idx_s)
        rec(4)
        ops.kv_gather(pk, pv, idx, pc.chunk, k_part=kp, v_part=vp)
        rec(5)
        ops.partial_draft_attn(pq, kp, vp, pkn, pvn, scale=pc.scale, out=dout, lse=dlse,
                               workspace=dws)
        rec(6)

    # The verify merge and the chunk importance depend on nothing of each other:
    # the timed step runs them as one launch (bit-identical results); the
    # per-kernel pass below keeps them apart so that each has its own time.
    def step_fused():
        ops.tree_verify_attn_partials(q, kc, vcache, kd, vd, parent, scale=vc.scale,
                                      o_part=o_part, l_part=l_part)
        ops.attn_merge_and_importance(o_part, l_part, pq, pk, pc.chunk, out=out, lse=lse, scale=pc.scale,
                                      scores=scores)
        ops.kv_topk_select(scores, pc.k, chunk_idx=idx, chunk_score=idx_s)
        ops.kv_gather(pk, pv, idx, pc.chunk, k_part=kp, v_part=vp)
        ops.partial_draft_attn(pq, kp, vp, pkn, pvn, scale=pc.scale, out=dout, lse=dlse,
                               workspace=dws)

    run_step = step if args.unfused else step_fused
    for _ in range(args.warmup):
        step()
        run_step()
    torch.cuda.synchronize()

    # With --graph the step is replayed as one HIP graph (nothing in it
    # allocates or clears memory); by default the launches are eager.
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()

    # timed region 1: K steps, wall clock between two syncs
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            run_step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps

    # timed region 2: the same K steps launched eagerly with HIP events between
    # the kernels (on torch's current stream, which every call launches on):
    # per-kernel durations for the roofline
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t2) * 1e3 / args.steps

    per = {n: [] for n in names}
    for ev in events:
        for j, n in enumerate(names):
            per[n].append(ev[j].elapsed_time(ev[j + 1]) * 1e3)   # us
    avg = {n: float(np.mean(v)) for n, v in per.items()}
    med = {n: float(np.median(v)) for n, v in per.items()}

    # ---- roofline of the dominant kernel (verify split-K) -------------------
    vis = 0
    par = vc.parent
    for t in range(T):           # |A(t)| summed over draft rows (the ancestor walk of the mask)
        a = t
        while a >= 0:
            vis += 1
            a = int(par[a])
    G = Hq // Hkv
    pairs = Hq * (T * L + vis)                  # (query row, visible key) pairs
    flops = 4.0 * D * pairs                     # QK^T and PV, 2 flops per MAC
    kv_bytes = 2.0 * Hkv * L * D * 2            # K and V of the cache, read once
    t_split = avg["verify_split"] * 1e-6
    achieved = flops / t_split / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(), "kernel": "verify split-K (attn_split_mfma_kernel)",
                "algorithmic_flops": flops, "algorithmic_bytes": kv_bytes,
                "hbm_GBs": round(kv_bytes / t_split / 1e9, 1),
                "hbm_frac": round(kv_bytes / t_split / 1e9 / HBM_PEAK_GBS, 4)}

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
        "config": {"workload": "llama3.1-8b layer, 102400-token bf16 KV cache: tree-verify of 120 drafts "
                               "([1,3,3,3] tree + 20 4-gram chains) + partial-KV refresh (4 queries, "
                               "64 of 1600 64-token chunks) + 4-query draft attention",
                   "T": T, "Hq": Hq, "Hkv": Hkv, "head_dim": D, "kv_len": L, "splits": S,
                   "chunk": pc.chunk, "topk": pc.k},
        "timing": ("graph replay of the step" if graph is not None else "eager launches") +
                  ("" if args.unfused else "; verify merge and chunk importance as one launch"),
        "eager_ms_per_step": round(eager_ms, 4),
        "verify_us": round(avg["verify_split"] + avg["verify_merge"], 2),
        "verify_hbm_frac": round(kv_bytes / ((avg["verify_split"] + avg["verify_merge"]) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_us_avg": {n: round(v, 2) for n, v in avg.items()},
        "kernel_us_median": {n: round(v, 2) for n, v in med.items()},
        "roofline": roofline,
    }

    res["accept_commit_us"] = time_accept_commit(vc, dev, args.steps)
    res["draft_tree_us"] = time_draft_tree(dev, args.steps)
    res["sample_us"] = time_sample(dev, args.steps)
    res["ngram_us"] = time_ngram(dev, args.steps)

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(vc, pc, args.cpu_heads, args.cpu_seconds)
    print(json.dumps(res), flush=True)


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


def time_sample(dev, reps):
    """Target tokens for the 121 verify rows over the LLaMA3.1 vocabulary:
    fp32 logits [121][128256], penalty 1.2 over 1024 tokens, temperature 1,
    min-p 0.1 (its own figure, not part of value)."""
    import torch
    from long_context_kv_ts_amd import inputs, ops
    c = inputs.make_sample(dtype="f32")
    logits = torch.from_numpy(c.logits).to(dev)
    hist, parent, dtok = (torch.from_numpy(a).to(dev) for a in (c.hist, c.parent, c.draft_tok))
    u = torch.from_numpy(c.u).to(dev)
    ws = ops.alloc_workspace(int(ops.lib().ts_sample_workspace(c.R, c.V)), dev)
    tok = torch.empty(c.R, dtype=torch.int32, device=dev)
    kw = dict(hist=hist, parent=parent, draft_tok=dtok, window=inputs.PENALTY_WINDOW, penalty=inputs.PENALTY,
              temperature=inputs.TEMPERATURE, min_p=inputs.MIN_P, u=u, tok=tok, workspace=ws)
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


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "verify_split_102400_hbm_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "long_context_kv_ts_amd", "csrc", f) for f in ("attn_mfma.hip", "common.h")]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the verify split kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by what the same counters read
    for a plain copy of known size; None if the kernel source has changed since."""
    try:
        kv = dict(line.split("=", 1) for line in open(TRAFFIC_FILE) if "=" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
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
        oracle.verify_attn_ref(vc.q, vc.k_cache, vc.v_cache, vc.k_draft, vc.v_draft, vc.parent,
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
