"""The whole step captured in a HIP graph and replayed: every replay must
reproduce the eager results bit for bit (the kernels are deterministic and
nothing in the step allocates or clears memory)."""
import numpy as np
import pytest
import torch

from long_context_kv_ts_amd import inputs, ops
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    say("[graph] verify + partial-KV step, 3 replays")
    dev = torch.device("cuda:0")
    c = inputs.make_verify("graph", dtype="bf16", Hq=32, Hkv=8, D=128, L=5000, seed=21, with_chains=True)
    p = inputs.make_partial(L=8192, seed=22)
    q, kc, vc, kd, vd = (to_dev(x, "bf16") for x in (c.q, c.k_cache, c.v_cache, c.k_draft, c.v_draft))
    par = to_dev(c.parent, "i32")
    pq, pk, pv, pkn, pvn = (to_dev(x, "bf16") for x in (p.q, p.k_cache, p.v_cache, p.k_new, p.v_new))
    S = ops.num_splits(c.T, c.Hq, c.Hkv, c.D, c.L, torch.bfloat16)
    o_part = torch.empty((S, c.T, c.Hq, c.D), dtype=torch.float32, device=dev)
    l_part = torch.empty((S, c.T, c.Hq), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((c.T, c.Hq), dtype=torch.float32, device=dev)
    scores = torch.empty((p.Hkv, p.n_chunks), dtype=torch.float32, device=dev)
    idx = torch.empty((p.Hkv, p.k), dtype=torch.int32, device=dev)
    val = torch.empty((p.Hkv, p.k), dtype=torch.float32, device=dev)
    kp = torch.empty((p.Hkv, p.k * p.chunk, p.D), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    dout = torch.empty_like(pq)
    dlse = torch.empty((p.R, p.Hq), dtype=torch.float32, device=dev)
    ws = ops.alloc_workspace(ops.lib().ts_partial_draft_attn_workspace(p.R, p.Hq, p.Hkv, p.D, p.k * p.chunk,
                                                                       ops.TS_BF16, 0), dev)

    def step():
        ops.tree_verify_attn_partials(q, kc, vc, kd, vd, par, scale=c.scale, o_part=o_part, l_part=l_part)
        ops.attn_merge(o_part, l_part, out=out, lse=lse)
        ops.kv_importance_score(pq, pk, p.chunk, scale=p.scale, scores=scores)
        ops.kv_topk_select(scores, p.k, chunk_idx=idx, chunk_score=val)
        ops.kv_gather(pk, pv, idx, p.chunk, k_part=kp, v_part=vp)
        ops.partial_draft_attn(pq, kp, vp, pkn, pvn, scale=p.scale, out=dout, lse=dlse, workspace=ws)

    results = (out, lse, scores, idx, val, kp, vp, dout, dlse)
    step()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for r in results:
            r.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "scores", "idx", "val", "kp", "vp", "dout", "dlse"), results, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"replay {rep}: {name}"


def test_graph_fused_step_and_sampling_replays_match_eager():
    """The benchmark's step (verify split with chunk importance, merge + top-k,
    gather + draft attention) and the target-token sampling with min-p and
    with top-p, captured once and replayed three times: the step bit for bit,
    the sampled tokens equal to the eager ones (the top-p counters and lists
    are reset by kernels of the call, not by memsets)."""
    say("[graph] fused step + sampling (min-p, top-p), 3 replays")
    dev = torch.device("cuda:0")
    p = inputs.make_partial(L=8192, seed=23)
    c = inputs.make_verify("graph_fused", dtype="bf16", Hq=p.Hq, Hkv=p.Hkv, D=p.D, L=p.L, seed=24, with_chains=True)
    q, kd, vd = (to_dev(x, "bf16") for x in (c.q, c.k_draft, c.v_draft))
    par = to_dev(c.parent, "i32")
    pq, pk, pv, pkn, pvn = (to_dev(x, "bf16") for x in (p.q, p.k_cache, p.v_cache, p.k_new, p.v_new))
    S = ops.num_splits(c.T, c.Hq, c.Hkv, c.D, p.L, torch.bfloat16)
    o_part = torch.empty((S, c.T, c.Hq, c.D), dtype=torch.float32, device=dev)
    l_part = torch.empty((S, c.T, c.Hq), dtype=torch.float32, device=dev)
    scores = torch.empty((p.Hkv, p.n_chunks), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((c.T, c.Hq), dtype=torch.float32, device=dev)
    idx = torch.empty((p.Hkv, p.k), dtype=torch.int32, device=dev)
    val = torch.empty((p.Hkv, p.k), dtype=torch.float32, device=dev)
    kp = torch.empty((p.Hkv, p.k * p.chunk, p.D), dtype=torch.bfloat16, device=dev)
    vp = torch.empty_like(kp)
    dout = torch.empty_like(pq)
    dlse = torch.empty((p.R, p.Hq), dtype=torch.float32, device=dev)
    dws = ops.alloc_workspace(ops.lib().ts_partial_draft_attn_workspace(p.R, p.Hq, p.Hkv, p.D, p.k * p.chunk,
                                                                        ops.TS_BF16, 0), dev)
    s = inputs.make_sample(dtype="f32", V=32000, seed=25)
    logits = torch.from_numpy(s.logits).to(dev)
    hist, sp, dtok = (torch.from_numpy(a).to(dev) for a in (s.hist, s.parent, s.draft_tok))
    u = torch.from_numpy(s.u).to(dev)
    sws = ops.alloc_workspace(int(ops.lib().ts_sample_workspace(s.R, s.V)), dev)
    tok_minp = torch.empty(s.R, dtype=torch.int32, device=dev)
    tok_topp = torch.empty(s.R, dtype=torch.int32, device=dev)
    tok_both = torch.empty(s.R, dtype=torch.int32, device=dev)
    kw = dict(hist=hist, parent=sp, draft_tok=dtok, window=inputs.PENALTY_WINDOW, penalty=inputs.PENALTY, u=u,
              workspace=sws)

    def step():
        ops.tree_verify_attn_partials_and_importance(q, pk, pv, kd, vd, par, pq, p.chunk, scale=c.scale,
                                                     imp_scale=p.scale, o_part=o_part, l_part=l_part, scores=scores)
        ops.attn_merge_and_topk(o_part, l_part, scores, p.k, out=out, lse=lse, chunk_idx=idx, chunk_score=val)
        ops.kv_gather_and_draft_attn(pk, pv, idx, p.chunk, pq, pkn, pvn, scale=p.scale, k_part=kp, v_part=vp,
                                     out=dout, lse=dlse, workspace=dws)
        ops.sample_tokens(logits, temperature=1.0, min_p=0.1, tok=tok_minp, **kw)
        ops.sample_tokens(logits, temperature=0.8, min_p=0.0, top_p=0.9, tok=tok_topp, **kw)
        ops.sample_tokens(logits, temperature=1.0, min_p=0.1, top_p=0.9, tok=tok_both, **kw)   # min-p binds

    names = ("out", "lse", "scores", "idx", "val", "kp", "vp", "dout", "dlse", "tok_minp", "tok_topp", "tok_both")
    results = (out, lse, scores, idx, val, kp, vp, dout, dlse, tok_minp, tok_topp, tok_both)
    step()
    torch.cuda.synchronize()
    eager = [r.clone() for r in results]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for r in results:
            r.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, results, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"replay {rep}: {name}"
