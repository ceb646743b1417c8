"""GPU: the calls that share one launch between two operations --
ts_attn_merge_and_importance, ts_attn_merge_and_topk and
ts_tree_verify_attn_partials_and_importance -- against the separate calls
(each pinned to the oracle in tests/test_gpu_verify.py and
tests/test_gpu_partial.py) and against the oracle at full size. The one-launch
paths run the same per-workgroup code as the separate kernels, so every output
must be bit-identical (the verify-with-importance kernel: to a stated
tolerance on the scores); shapes outside them take the separate launches and
must be too."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say
from long_context_kv_ts_amd import ops
from oracle import partial_kv

pytestmark = pytest.mark.gpu


def _inputs(seed, S, T, Hq_v, Dv, R, Hq, Hkv, D, L, empty_splits=False):
    g = torch.Generator(device="cpu").manual_seed(seed)
    o_part = torch.randn((S, T, Hq_v, Dv), generator=g).to(DEV)
    l_part = (torch.randn((S, T, Hq_v), generator=g) * 3).to(DEV)
    if empty_splits:
        l_part[::3, :, 1] = -float("inf")                 # splits that saw no key of a row
        l_part[:, 0, 0] = -float("inf")                   # a row with no key at all
    q = torch.randn((R, Hq, D), generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn((Hkv, L, D), generator=g).to(torch.bfloat16).to(DEV)
    return o_part, l_part, q, k


@pytest.mark.parametrize("case", [
    # S, T, Hq_v, Dv, R, Hq, Hkv, D, L, chunk, out dtype
    dict(S=16, T=120, Hq_v=32, Dv=128, R=4, Hq=32, Hkv=8, D=128, L=64 * 101, chunk=64, odt=torch.bfloat16),
    dict(S=16, T=7, Hq_v=28, Dv=128, R=4, Hq=28, Hkv=4, D=128, L=64 * 40, chunk=64, odt=torch.bfloat16),
    dict(S=9, T=5, Hq_v=64, Dv=128, R=4, Hq=64, Hkv=4, D=128, L=64 * 33, chunk=64, odt=torch.float32),
    dict(S=20, T=120, Hq_v=32, Dv=128, R=4, Hq=32, Hkv=8, D=128, L=64 * 50, chunk=64, odt=torch.bfloat16),
    dict(S=16, T=120, Hq_v=32, Dv=64, R=4, Hq=32, Hkv=8, D=64, L=64 * 50, chunk=64, odt=torch.bfloat16),
    dict(S=16, T=120, Hq_v=32, Dv=128, R=4, Hq=32, Hkv=8, D=128, L=32 * 77, chunk=32, odt=torch.bfloat16),
], ids=["bench-shape", "G7", "rows64-f32", "S20-two-launches", "D64-two-launches", "chunk32-two-launches"])
@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32-partials", "bf16-partials"])
def test_bit_identical_to_separate_calls(case, pdt):
    c = dict(case)
    odt, chunk = c.pop("odt"), c.pop("chunk")
    say(f"fused merge+importance {case} partials {pdt}")
    o_part, l_part, q, k = _inputs(5, **c, empty_splits=True)
    o_part = o_part.to(pdt)
    out_a, lse_a = ops.attn_merge(o_part, l_part, out_dtype=odt)
    scores_a = ops.kv_importance_score(q, k, chunk, scale=0.09)
    out_b, lse_b, scores_b = ops.attn_merge_and_importance(o_part, l_part, q, k, chunk, out_dtype=odt, scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16) if odt == torch.bfloat16 else out_a.view(torch.int32),
                       out_b.view(torch.int16) if odt == torch.bfloat16 else out_b.view(torch.int32))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    assert torch.equal(scores_a.view(torch.int32), scores_b.view(torch.int32))
    assert np.isfinite(scores_b.cpu().numpy()).all()


def test_repeated_calls_reuse_outputs():
    """Outputs handed in are overwritten in full on every call."""
    o_part, l_part, q, k = _inputs(6, 16, 120, 32, 128, 4, 32, 8, 128, 64 * 64)
    out, lse, scores = ops.attn_merge_and_importance(o_part, l_part, q, k, 64)
    ref = (out.clone(), lse.clone(), scores.clone())
    out.fill_(7.0)
    lse.fill_(7.0)
    scores.fill_(7.0)
    ops.attn_merge_and_importance(o_part, l_part, q, k, 64, out=out, lse=lse, scores=scores)
    torch.cuda.synchronize()
    for a, b in zip(ref, (out, lse, scores)):
        assert torch.equal(a, b)


def test_bench_launch_at_full_size_against_the_oracle():
    """The one launch a decode step times, at its real size: the verify split
    partials of the LLaMA3.1-8B layer over 102,400 cached tokens (16 splits,
    3840 merged rows) together with the chunk importance of the 102,400-token
    partial-KV workload (8 KV heads x 1600 chunks of 64 tokens; 6400 chunk-pair
    workgroups). out and lse are compared with the oracle's tree-verify
    attention and the scores with its importance, element by element."""
    import oracle
    from gpu_util import check_attn, to_dev
    from long_context_kv_ts_amd import inputs

    vc = inputs.workload("llama8b_100k")
    pc = inputs.workload("partial_100k")
    say("[fused full size] llama8b_100k partials + partial_100k importance")
    o_part, l_part = ops.tree_verify_attn_partials(
        to_dev(vc.q, "bf16"), to_dev(vc.k_cache, "bf16"), to_dev(vc.v_cache, "bf16"), to_dev(vc.k_draft, "bf16"),
        to_dev(vc.v_draft, "bf16"), to_dev(vc.parent, "i32"), scale=vc.scale)
    # one wave per merged row covers 16 splits: the one-launch path, not the fallback
    assert o_part.shape[0] == 16
    pq, pk = to_dev(pc.q, "bf16"), to_dev(pc.k_cache, "bf16")
    out, lse, scores = ops.attn_merge_and_importance(o_part, l_part, pq, pk, pc.chunk, scale=pc.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn_ref(vc.q, vc.k_cache, vc.v_cache, vc.k_draft, vc.v_draft, vc.parent,
                                    vc.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "fused merge vs verify oracle")
    rs = oracle.importance_ref(pc.q, pc.k_cache, pc.scale, pc.chunk, "bf16")
    got = scores.cpu().numpy().astype(np.float64)
    err = np.abs(got - rs).max()
    say(f"  importance: max|d| {err:.3e} (max|ref| {np.abs(rs).max():.3e})")
    assert got.shape == rs.shape == (8, 1600)
    assert err <= 1e-5 * np.abs(rs).max()


# ---------------------------------------------------------------------------
# verify split partials and chunk importance of the same cache in one launch
# ---------------------------------------------------------------------------
def _dev(a, dt):
    from gpu_util import to_dev
    return to_dev(a, dt)


def _partials_and_scores(c, q_rec, chunk, imp_scale, num_splits=0, part_dtype=torch.float32):
    dt = c.dtype
    args = (_dev(c.q, dt), _dev(c.k_cache, dt), _dev(c.v_cache, dt), _dev(c.k_draft, dt), _dev(c.v_draft, dt),
            _dev(c.parent, "i32"))
    qr = _dev(q_rec, dt)
    o1, l1, s1 = ops.tree_verify_attn_partials_and_importance(*args, qr, chunk, scale=c.scale, imp_scale=imp_scale,
                                                             num_splits=num_splits, part_dtype=part_dtype)
    o2, l2 = ops.tree_verify_attn_partials(*args, scale=c.scale, num_splits=num_splits, part_dtype=part_dtype)
    s2 = ops.kv_importance_score(qr, args[1], chunk, scale=imp_scale)
    torch.cuda.synchronize()
    return (o1, l1, s1), (o2, l2, s2)


def _check_same(fused, sep, label, imp_rel=1e-5):
    (o1, l1, s1), (o2, l2, s2) = fused, sep
    iv = torch.int16 if o1.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(o1.view(iv), o2.view(iv)), f"{label}: partials differ"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"{label}: partial lse differ"
    a, b = s1.cpu().numpy().astype(np.float64), s2.cpu().numpy().astype(np.float64)
    err = np.abs(a - b).max()
    say(f"  {label}: partials bit-identical; scores max|d| {err:.3e} (max {np.abs(b).max():.3e})")
    assert err <= imp_rel * np.abs(b).max()


def test_partials_and_importance_full_size_against_the_oracle():
    """One decode step's cache: the partial-KV workload's 102,400-token cache
    (8 boosted chunks per KV head) verified for the 120 drafts of the
    LLaMA3.1-8B tree + chains and scored for its 4 recent queries in one
    launch; merged output and lse against the oracle's verify attention, the
    scores against its importance, and both against the separate calls."""
    import oracle
    from gpu_util import check_attn
    from long_context_kv_ts_amd import inputs

    vc = inputs.workload("llama8b_100k")
    pc = inputs.workload("partial_100k")
    vc.k_cache, vc.v_cache = pc.k_cache, pc.v_cache           # one cache for the whole step
    say("[verify+importance full size] partial_100k cache, llama8b_100k drafts")
    fused, sep = _partials_and_scores(vc, pc.q, pc.chunk, pc.scale)
    _check_same(fused, sep, "102400")
    o, l, s = fused
    out, lse = ops.attn_merge(o, l)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn_ref(vc.q, vc.k_cache, vc.v_cache, vc.k_draft, vc.v_draft, vc.parent, vc.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "fused split + merge vs verify oracle")
    rs = oracle.importance_ref(pc.q, pc.k_cache, pc.scale, pc.chunk, "bf16")
    err = np.abs(s.cpu().numpy().astype(np.float64) - rs).max()
    say(f"  importance vs oracle: max|d| {err:.3e} (max|ref| {np.abs(rs).max():.3e})")
    assert err <= 1e-5 * np.abs(rs).max()
    idx, _ = ops.kv_topk_select(s, pc.k)
    ref_idx, _ = oracle.topk_ref(s.cpu().numpy().astype(np.float64), pc.k)
    assert (idx.cpu().numpy() == ref_idx).all(), "top-k of the fused scores"


@pytest.mark.parametrize("case", [
    # Hq, Hkv, T, L, R: fused shapes (the last row group ends in an empty wave) and fallbacks
    dict(Hq=32, Hkv=8, T=120, L=64 * 101, R=4),     # 480 rows: fused
    dict(Hq=16, Hkv=8, T=100, L=64 * 77, R=4),      # G = 2, 200 rows: fused
    dict(Hq=4, Hkv=4, T=200, L=64 * 50, R=4),       # G = 1, 200 rows: fused
    dict(Hq=32, Hkv=8, T=120, L=64 * 40, R=8),      # R*G = 32: fused
    dict(Hq=32, Hkv=8, T=60, L=64 * 40, R=4),       # 240 rows: last wave holds rows -> two launches
    dict(Hq=4, Hkv=4, T=120, L=64 * 40, R=4),       # MHA 120 rows (128-row form) -> two launches
    dict(Hq=28, Hkv=4, T=40, L=64 * 33, R=4),       # G = 7 -> two launches
    dict(Hq=32, Hkv=8, T=300, L=64 * 20, R=4),      # more than 256 drafts -> two launches
])
@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32-partials", "bf16-partials"])
def test_partials_and_importance_shapes(case, pdt):
    from long_context_kv_ts_amd import inputs
    c = inputs.make_verify("vi", dtype="bf16", Hq=case["Hq"], Hkv=case["Hkv"], D=128, L=case["L"], seed=31,
                           with_chains=False,
                           parent=np.array([-1 if t % 7 == 0 else t - 1 for t in range(case["T"])], np.int32))
    rng = np.random.default_rng(32)
    q_rec = inputs.f32_to_bf16_bits(rng.standard_normal((case["R"], case["Hq"], 128)).astype(np.float32))
    say(f"[verify+importance] {case} partials {pdt}")
    fused, sep = _partials_and_scores(c, q_rec, 64, 0.0884, part_dtype=pdt)
    _check_same(fused, sep, str(case))


@pytest.mark.parametrize("ns", [1, 3, 16, 40])
def test_partials_and_importance_split_counts(ns):
    """Splits start on 64-token chunks whatever their count."""
    from long_context_kv_ts_amd import inputs
    c = inputs.make_verify("vs", dtype="bf16", Hq=32, Hkv=8, D=128, L=64 * 123, seed=33, with_chains=True)
    rng = np.random.default_rng(34)
    q_rec = inputs.f32_to_bf16_bits(rng.standard_normal((4, 32, 128)).astype(np.float32))
    say(f"[verify+importance] splits={ns}")
    fused, sep = _partials_and_scores(c, q_rec, 64, 0.0884, num_splits=ns)
    _check_same(fused, sep, f"splits={ns}")


# ---------------------------------------------------------------------------
# ts_attn_merge_and_topk: the merge and the chunk top-k in one grid.

def _scores(seed, Hkv, n, ties=False):
    g = torch.Generator(device="cpu").manual_seed(seed)
    s = torch.randn((Hkv, n), generator=g)
    if ties:
        s = torch.round(s * 4) / 4                        # many equal scores
        s[:, : n // 4] = 0.5
    return s.to(DEV)


@pytest.mark.parametrize("case", [
    # S, T, Hq_v, Dv, Hkv, n_chunks, k, out dtype
    dict(S=16, T=120, Hq_v=32, Dv=128, Hkv=8, n=1600, k=64, odt=torch.bfloat16),
    dict(S=16, T=120, Hq_v=32, Dv=128, Hkv=8, n=2048, k=2048, odt=torch.bfloat16),
    dict(S=9, T=5, Hq_v=64, Dv=128, Hkv=4, n=3000, k=100, odt=torch.float32),
    dict(S=1, T=3, Hq_v=8, Dv=128, Hkv=2, n=1, k=1, odt=torch.bfloat16),
    dict(S=16, T=120, Hq_v=32, Dv=128, Hkv=8, n=20000, k=313, odt=torch.bfloat16),
    dict(S=20, T=120, Hq_v=32, Dv=128, Hkv=8, n=1600, k=64, odt=torch.bfloat16),
    dict(S=16, T=120, Hq_v=32, Dv=64, Hkv=8, n=1600, k=64, odt=torch.bfloat16),
], ids=["bench-shape", "k-equals-n", "streamed-f32", "tiny", "n20000", "S20-two-launches", "D64-two-launches"])
@pytest.mark.parametrize("ties", [False, True], ids=["distinct", "ties"])
@pytest.mark.parametrize("pdt", [torch.float32, torch.bfloat16], ids=["f32-partials", "bf16-partials"])
def test_merge_topk_bit_identical_to_separate_calls(case, ties, pdt):
    c = dict(case)
    say(f"fused merge+topk {case} ties={ties} partials {pdt}")
    o_part, l_part, _, _ = _inputs(7, c["S"], c["T"], c["Hq_v"], c["Dv"], 1, 1, 1, 64, 64, empty_splits=True)
    o_part = o_part.to(pdt)
    scores = _scores(8, c["Hkv"], c["n"], ties)
    out_a, lse_a = ops.attn_merge(o_part, l_part, out_dtype=c["odt"])
    idx_a, val_a = ops.kv_topk_select(scores, c["k"])
    out_b, lse_b, idx_b, val_b = ops.attn_merge_and_topk(o_part, l_part, scores, c["k"], out_dtype=c["odt"])
    torch.cuda.synchronize()
    iv = torch.int16 if c["odt"] == torch.bfloat16 else torch.int32
    assert torch.equal(out_a.view(iv), out_b.view(iv))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    assert torch.equal(idx_a, idx_b)
    assert torch.equal(val_a.view(torch.int32), val_b.view(torch.int32))
    # the top-k half against the oracle on its own too
    ref_idx, _ = partial_kv.topk_ref(scores.cpu().numpy().astype(np.float64), c["k"])
    np.testing.assert_array_equal(idx_b.cpu().numpy(), ref_idx)


def test_merge_topk_without_scores_and_reused_outputs():
    o_part, l_part, _, _ = _inputs(9, 16, 120, 32, 128, 1, 1, 1, 64, 64)
    scores = _scores(10, 8, 1600)
    out, lse, idx, val = ops.attn_merge_and_topk(o_part, l_part, scores, 64)
    ref = (out.clone(), lse.clone(), idx.clone(), val.clone())
    out.fill_(7.0)
    lse.fill_(7.0)
    idx.fill_(-1)
    ops.attn_merge_and_topk(o_part, l_part, scores, 64, out=out, lse=lse, chunk_idx=idx, want_scores=False)
    torch.cuda.synchronize()
    for a, b in zip(ref[:3], (out, lse, idx)):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# ts_kv_gather_and_draft_attn: the gather done by the draft pass.

def _gather_draft_inputs(seed, Hkv, L, D, Tq, Hq, k, chunk, dtype=torch.bfloat16, bad_idx=False):
    g = torch.Generator(device="cpu").manual_seed(seed)
    kc = torch.randn((Hkv, L, D), generator=g).to(dtype).to(DEV)
    vc = torch.randn((Hkv, L, D), generator=g).to(dtype).to(DEV)
    idx = torch.stack([torch.randperm(L // chunk, generator=g)[:k].sort().values for _ in range(Hkv)])
    if bad_idx:
        idx[0, 1] = -1                    # out of range: a zero chunk in both paths
        idx[-1, -1] = L // chunk
    q = torch.randn((Tq, Hq, D), generator=g).to(dtype).to(DEV)
    kn = torch.randn((Hkv, Tq, D), generator=g).to(dtype).to(DEV)
    vn = torch.randn((Hkv, Tq, D), generator=g).to(dtype).to(DEV)
    return kc, vc, idx.to(torch.int32).to(DEV), q, kn, vn


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", [
    # Hkv, L, D, Tq, Hq, k, chunk, splits, dtype
    dict(Hkv=8, L=102400, D=128, Tq=4, Hq=32, k=64, chunk=64, ns=0, dt=torch.bfloat16),
    dict(Hkv=8, L=8192, D=128, Tq=4, Hq=32, k=64, chunk=64, ns=7, dt=torch.bfloat16),
    dict(Hkv=4, L=16384, D=128, Tq=1, Hq=28, k=40, chunk=64, ns=0, dt=torch.bfloat16),
    dict(Hkv=8, L=8192, D=64, Tq=2, Hq=32, k=33, chunk=64, ns=0, dt=torch.bfloat16),
    dict(Hkv=8, L=8192, D=128, Tq=4, Hq=32, k=64, chunk=32, ns=0, dt=torch.bfloat16),
    dict(Hkv=8, L=8192, D=128, Tq=4, Hq=32, k=16, chunk=64, ns=0, dt=torch.float32),
    dict(Hkv=2, L=4096, D=128, Tq=16, Hq=16, k=8, chunk=64, ns=0, dt=torch.bfloat16),
], ids=["bench-shape", "splits7", "G7-Tq1", "D64", "chunk32-two-calls", "f32-two-calls", "mfma-path-two-calls"])
def test_gather_draft_bit_identical_to_separate_calls(case):
    c = dict(case)
    say(f"gather+draft {case}")
    kc, vc, idx, q, kn, vn = _gather_draft_inputs(11, c["Hkv"], c["L"], c["D"], c["Tq"], c["Hq"], c["k"],
                                                  c["chunk"], c["dt"], bad_idx=True)
    kp_a, vp_a = ops.kv_gather(kc, vc, idx, c["chunk"])
    out_a, lse_a = ops.partial_draft_attn(q, kp_a, vp_a, kn, vn, scale=0.088, num_splits=c["ns"])
    kp_b, vp_b, out_b, lse_b = ops.kv_gather_and_draft_attn(kc, vc, idx, c["chunk"], q, kn, vn, scale=0.088,
                                                            num_splits=c["ns"])
    torch.cuda.synchronize()
    assert torch.equal(_bits(kp_a), _bits(kp_b))
    assert torch.equal(_bits(vp_a), _bits(vp_b))
    assert torch.equal(_bits(out_a), _bits(out_b))
    assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
    assert torch.isfinite(out_b.float()).all()


def test_gather_draft_full_size_against_the_oracle():
    """The launch the decode step times, at its real size: 64 chunks of 64
    tokens per KV head chosen from a 102,400-token LLaMA3.1-8B cache, gathered
    and attended by 4 draft tokens, against the oracle's gather (bit-exact)
    and draft attention (element by element)."""
    from long_context_kv_ts_amd import inputs
    from gpu_util import check_attn, to_dev
    import oracle
    p = inputs.make_partial(L=102400, seed=3)
    rng = np.random.default_rng(5)
    gidx = np.stack([np.sort(rng.choice(p.L // p.chunk, p.k, replace=False)) for _ in range(p.Hkv)]).astype(np.int32)
    say("gather+draft full size vs oracle")
    kp, vp, out, lse = ops.kv_gather_and_draft_attn(
        to_dev(p.k_cache, "bf16"), to_dev(p.v_cache, "bf16"), torch.from_numpy(gidx).to(DEV), p.chunk,
        to_dev(p.q, "bf16"), to_dev(p.k_new, "bf16"), to_dev(p.v_new, "bf16"), scale=p.scale)
    torch.cuda.synchronize()
    rkp, rvp = oracle.gather_ref(p.k_cache, p.v_cache, gidx, p.chunk)
    np.testing.assert_array_equal(kp.view(torch.int16).cpu().numpy().view(np.uint16), rkp)
    np.testing.assert_array_equal(vp.view(torch.int16).cpu().numpy().view(np.uint16), rvp)
    ro, rl = oracle.draft_attn_ref(p.q, rkp, rvp, p.k_new, p.v_new, p.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "gathered draft attention")


def test_bench_step_at_full_size_against_the_oracle():
    """The decode step exactly as the benchmark times it -- four kernels through
    the three combined calls (bf16 split partials), on the 102,400-token LLaMA3.1-8B cache with its 4
    recent queries and the 120-draft forest -- against the oracle: verify output
    and lse element by element, chunk scores within 1e-5, the top-64 bit-exact on
    the GPU's own scores and within the near-tie rule on the oracle's, the partial
    cache bit-exact, the draft attention element by element."""
    from long_context_kv_ts_amd import inputs
    from gpu_util import check_attn, to_dev
    import oracle
    from test_gpu_partial import topk_matches_with_near_tie_rule
    pc = inputs.workload("partial_100k")
    vc = inputs.workload("llama8b_100k", L=64)          # the same drafts and forest, without its own cache
    say("bench step at full size vs oracle")
    kc, v_c = to_dev(pc.k_cache, "bf16"), to_dev(pc.v_cache, "bf16")
    q, kd, vd = to_dev(vc.q, "bf16"), to_dev(vc.k_draft, "bf16"), to_dev(vc.v_draft, "bf16")
    parent = torch.from_numpy(vc.parent).to(DEV)
    pq = to_dev(pc.q, "bf16")
    o_part, l_part, scores = ops.tree_verify_attn_partials_and_importance(
        q, kc, v_c, kd, vd, parent, pq, pc.chunk, scale=vc.scale, imp_scale=pc.scale, part_dtype=torch.bfloat16)
    out, lse, idx, _ = ops.attn_merge_and_topk(o_part, l_part, scores, pc.k)
    kp, vp, dout, dlse = ops.kv_gather_and_draft_attn(kc, v_c, idx, pc.chunk, pq, to_dev(pc.k_new, "bf16"),
                                                      to_dev(pc.v_new, "bf16"), scale=pc.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.verify_attn_ref(vc.q, pc.k_cache, pc.v_cache, vc.k_draft, vc.v_draft, vc.parent, vc.scale,
                                    "bf16")
    check_attn(out, lse, ro, rl, "bf16", "step verify")
    ref_s = oracle.importance_ref(pc.q, pc.k_cache, pc.scale, pc.chunk, "bf16")
    gs = scores.cpu().numpy().astype(np.float64)
    assert np.abs(gs - ref_s).max() <= 1e-5 * np.abs(ref_s).max()
    gidx = idx.cpu().numpy()
    same_prec, _ = oracle.topk_ref(gs, pc.k)
    np.testing.assert_array_equal(gidx, same_prec)
    topk_matches_with_near_tie_rule(gidx, ref_s, pc.k)
    rkp, rvp = oracle.gather_ref(pc.k_cache, pc.v_cache, gidx, pc.chunk)
    np.testing.assert_array_equal(kp.view(torch.int16).cpu().numpy().view(np.uint16), rkp)
    np.testing.assert_array_equal(vp.view(torch.int16).cpu().numpy().view(np.uint16), rvp)
    rd, rdl = oracle.draft_attn_ref(pc.q, rkp, rvp, pc.k_new, pc.v_new, pc.scale, "bf16")
    check_attn(dout, dlse, rd, rdl, "bf16", "step draft attention")
