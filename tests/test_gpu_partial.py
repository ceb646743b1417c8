"""GPU parity of the partial-KV step -- ts_kv_importance_score, ts_kv_topk_select,
ts_kv_gather, ts_partial_draft_attn -- against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from long_context_kv_ts_amd import inputs, ops
import oracle
from gpu_util import check_attn, say, to_dev, to_host

pytestmark = pytest.mark.gpu

# importance: fp32 sums of bf16 products (exact) over chunk*R terms
SCORE_REL = 1e-5
NEAR_TIE = 1e-4     # relative gap at the k-th boundary below which the set may differ inside the band


def topk_matches_with_near_tie_rule(got_idx, ref_scores, k):
    """Same set as the oracle's, except inside the near-tie band at the k-th
    boundary when the oracle's relative gap there is below NEAR_TIE."""
    for g in range(ref_scores.shape[0]):
        s = ref_scores[g]
        order = np.lexsort((np.arange(len(s)), -s))
        ref_set = set(order[:k].tolist())
        got = got_idx[g].tolist()
        assert len(set(got)) == k and got == sorted(got), f"head {g}: not k distinct ascending"
        sk = s[order[k - 1]]
        sk1 = s[order[k]] if k < len(s) else -np.inf
        gap = (sk - sk1) / abs(sk)
        if gap >= NEAR_TIE:
            assert set(got) == ref_set, f"head {g}: set differs (gap {gap:.2e})"
        else:
            band = set(np.nonzero(np.abs(s - sk) <= NEAR_TIE * abs(sk))[0].tolist())
            assert set(got) - band == ref_set - band, f"head {g}: differs outside the near-tie band"


_cache = {}


def partial_case(L=None, seed=None):
    key = (L, seed)
    if key not in _cache:
        _cache.clear()
        _cache[key] = inputs.make_partial(L=102400 if L is None else L, seed=3 if seed is None else seed)
    return _cache[key]


@pytest.mark.parametrize("L", [102400, 8192])
def test_partial_step_full(L):
    say(f"[partial step] L={L}")
    check_partial_step(partial_case(L))


@pytest.mark.parametrize("Hq,Hkv", [(28, 4), (12, 2), (40, 8)])
def test_partial_step_qwen_group_sizes(Hq, Hkv):
    """Qwen2.5-7B (28 query heads, 4 KV heads: G = 7), -1.5B (G = 6) and -14B (G = 5)
    group sizes: the importance max then spans groups that are not a power of two."""
    say(f"[partial step] Hq={Hq} Hkv={Hkv} G={Hq // Hkv}")
    check_partial_step(inputs.make_partial(f"qwen_g{Hq // Hkv}", Hq=Hq, Hkv=Hkv, L=16384, seed=Hq))


def check_partial_step(p):
    q, kc, vc = to_dev(p.q, "bf16"), to_dev(p.k_cache, "bf16"), to_dev(p.v_cache, "bf16")
    scores = ops.kv_importance_score(q, kc, p.chunk, scale=p.scale)
    idx, val = ops.kv_topk_select(scores, p.k)
    kp, vp = ops.kv_gather(kc, vc, idx, p.chunk)
    out, lse = ops.partial_draft_attn(q, kp, vp, to_dev(p.k_new, "bf16"), to_dev(p.v_new, "bf16"), scale=p.scale)
    torch.cuda.synchronize()

    # a5 importance: element by element
    ref_s = oracle.importance_ref(p.q, p.k_cache, p.scale, p.chunk, "bf16")
    gs = scores.cpu().numpy().astype(np.float64)
    err = np.abs(gs - ref_s).max()
    say(f"  importance max|d| {err:.3e} (max|ref| {np.abs(ref_s).max():.3e})")
    assert err <= SCORE_REL * np.abs(ref_s).max()

    # a6 top-k: bit-exact given the same fp32 scores; near-tie rule vs fp64 scores
    gidx = idx.cpu().numpy()
    same_prec_idx, same_prec_val = oracle.topk_ref(gs, p.k)
    np.testing.assert_array_equal(gidx, same_prec_idx)
    np.testing.assert_array_equal(val.cpu().numpy(), same_prec_val.astype(np.float32))
    topk_matches_with_near_tie_rule(gidx, ref_s, p.k)
    for g in range(p.Hkv):
        assert set(p.boosted[g]).issubset(set(gidx[g])), "a 3x-key chunk was not selected"

    # a7 gather: bit-exact for the GPU's own indices
    rkp, rvp = oracle.gather_ref(p.k_cache, p.v_cache, gidx, p.chunk)
    np.testing.assert_array_equal(kp.view(torch.int16).cpu().numpy().view(np.uint16), rkp)
    np.testing.assert_array_equal(vp.view(torch.int16).cpu().numpy().view(np.uint16), rvp)

    # a8 draft attention over the gathered cache
    ro, rl = oracle.draft_attn_ref(p.q, rkp, rvp, p.k_new, p.v_new, p.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "draft attention")


def test_topk_ties_and_edges():
    say("[topk] ties, k = n, k = 1")
    rng = np.random.default_rng(0)
    for n, k in ((1600, 64), (1600, 1600), (1600, 1), (7, 3), (65536, 64), (5000, 4096),
                 (4096, 64), (4096, 65), (1024, 64), (1025, 33), (64, 64), (2048, 63)):
        s = np.round(rng.standard_normal((3, n)), 2).astype(np.float32)   # many exact ties
        s[1] = 0.5                                                        # all equal
        s[2, ::3] = -0.0
        s[2, 1::3] = 0.0
        idx, val = ops.kv_topk_select(torch.from_numpy(s).cuda(), k)
        torch.cuda.synchronize()
        ref_idx, ref_val = oracle.topk_ref(s.astype(np.float64), k)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx, err_msg=f"n={n} k={k}")
        np.testing.assert_array_equal(val.cpu().numpy(), np.take_along_axis(s, ref_idx, 1),
                                      err_msg=f"values n={n} k={k}")


def test_topk_narrow_ranges_and_low_bit_keys():
    """Scores that share sign, exponent and leading mantissa bits (as one head's
    importance scores do), keys that differ only in their last mantissa bits, and
    sizes around one wave, one 1024-thread round and the 4096-element limit of
    the register-resident variant."""
    say("[topk] narrow ranges, low-bit keys, variant boundaries")
    rng = np.random.default_rng(5)
    for n in (1, 63, 64, 65, 1023, 1024, 1025, 1600, 2047, 2048, 2049, 4095, 4096, 4097):
        for kind in range(3):
            if kind == 0:
                s = 0.09 + 0.014 * rng.standard_normal((4, n))
            elif kind == 1:
                s = np.float32(0.3) + np.float32(3e-8) * rng.integers(0, 6, (4, n))
            else:
                s = np.float32(-1.5) - np.float32(1e-7) * rng.integers(0, 40, (4, n))
            s = s.astype(np.float32)
            for k in sorted({1, min(n, 64), min(n, 65), n}):
                idx, val = ops.kv_topk_select(torch.from_numpy(s).cuda(), k)
                torch.cuda.synchronize()
                ref_idx, _ = oracle.topk_ref(s.astype(np.float64), k)
                np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx, err_msg=f"n={n} k={k} kind={kind}")
                np.testing.assert_array_equal(val.cpu().numpy(), np.take_along_axis(s, ref_idx, 1))


def test_topk_negative_and_infinite_scores():
    s = np.array([[-1.0, -np.inf, 3.0, np.inf, -2.5, 3.0, -0.0, 0.0]], np.float32)
    idx, _ = ops.kv_topk_select(torch.from_numpy(s).cuda(), 4)
    torch.cuda.synchronize()
    ref, _ = oracle.topk_ref(s.astype(np.float64), 4)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)


def test_importance_shapes():
    say("[importance] shapes")
    rng = np.random.default_rng(1)
    for (R, Hq, Hkv, D, L, chunk, dt) in ((4, 32, 8, 128, 4096, 64, "bf16"),
                                          (4, 32, 32, 128, 2048, 64, "bf16"),   # MHA
                                          (2, 16, 2, 64, 1920, 48, "bf16"),     # G=8, ragged 16-key block
                                          (3, 8, 2, 128, 1000, 40, "bf16"),
                                          (4, 28, 4, 128, 4096, 64, "bf16"),    # G=7 (Qwen2.5-7B)
                                          (4, 12, 2, 128, 2048, 64, "bf16"),    # G=6
                                          (4, 40, 8, 64, 1920, 40, "bf16"),     # G=5, chunk 40: ragged last 16-key block
                                          (5, 36, 12, 128, 1000, 40, "bf16"),   # G=3, R=5
                                          (5, 24, 2, 128, 2048, 64, "bf16"),    # G=12: 60 rows, 4 row blocks
                                          (4, 15, 1, 64, 1024, 64, "bf16"),     # G=15
                                          (4, 28, 4, 64, 1024, 64, "f32")):
        q = rng.standard_normal((R, Hq, D)).astype(np.float32)
        k = (rng.standard_normal((Hkv, L, D)) / np.sqrt(D)).astype(np.float32)
        if dt == "bf16":
            q, k = inputs.f32_to_bf16_bits(q), inputs.f32_to_bf16_bits(k)
        s = ops.kv_importance_score(to_dev(q, dt), to_dev(k, dt), chunk, scale=D ** -0.5)
        torch.cuda.synchronize()
        ref = oracle.importance_ref(q, k, D ** -0.5, chunk, dt)
        err = np.abs(s.cpu().numpy() - ref).max()
        say(f"  R={R} Hq={Hq} Hkv={Hkv} D={D} L={L} chunk={chunk} {dt}: {err:.2e}")
        assert err <= SCORE_REL * np.abs(ref).max()


def test_gather_out_of_range_index_zero_fills():
    kc = torch.arange(2 * 256 * 64, dtype=torch.int16).view(torch.bfloat16).reshape(2, 256, 64).cuda()
    vc = (kc.view(torch.int16) + 1).view(torch.bfloat16)
    idx = torch.tensor([[3, 99, 0], [-1, 1, 2]], dtype=torch.int32).cuda()   # 4 chunks of 64 per head
    kp, vp = ops.kv_gather(kc, vc, idx, 64)
    torch.cuda.synchronize()
    assert torch.equal(kp[0, :64].view(torch.int16), kc[0, 192:256].view(torch.int16))
    assert (kp[0, 64:128].view(torch.int16) == 0).all()
    assert (vp[1, :64].view(torch.int16) == 0).all()
    assert torch.equal(vp[1, 128:192].view(torch.int16), vc[1, 128:192].view(torch.int16))


@pytest.mark.parametrize("shape", [dict(Hq=32, Hkv=8, D=128), dict(Hq=32, Hkv=32, D=128),
                                   dict(Hq=8, Hkv=1, D=64)])
def test_draft_attention_shapes(shape):
    say(f"[draft attn] {shape}")
    rng = np.random.default_rng(2)
    Tq, P = 4, 4096
    Hq, Hkv, D = shape["Hq"], shape["Hkv"], shape["D"]
    f = lambda *s, sd=1.0: inputs.f32_to_bf16_bits((rng.standard_normal(s) * sd).astype(np.float32))
    q, kp, vp = f(Tq, Hq, D), f(Hkv, P, D, sd=D ** -0.5), f(Hkv, P, D, sd=D ** -0.5)
    kn, vn = f(Hkv, Tq, D, sd=D ** -0.5), f(Hkv, Tq, D, sd=D ** -0.5)
    out, lse = ops.partial_draft_attn(*(to_dev(a, "bf16") for a in (q, kp, vp, kn, vn)), scale=D ** -0.5)
    torch.cuda.synchronize()
    ro, rl = oracle.draft_attn_ref(q, kp, vp, kn, vn, D ** -0.5, "bf16")
    check_attn(out, lse, ro, rl, "bf16", str(shape))


@pytest.mark.parametrize("Tq,Hq,Hkv,D,P", [(4, 32, 8, 128, 4096), (4, 32, 8, 128, 1000), (1, 8, 2, 128, 777),
                                          (3, 16, 4, 64, 300), (16, 16, 16, 128, 2100), (2, 4, 4, 128, 64)])
def test_small_row_kernel_shapes(Tq, Hq, Hkv, D, P):
    """KV heads with at most 16 grouped rows (wave-per-split kernel), ragged lengths."""
    say(f"[small rows] Tq={Tq} Hq={Hq} Hkv={Hkv} D={D} P={P}")
    rng = np.random.default_rng(Tq * 1000 + P)
    f = lambda *s, sd=1.0: inputs.f32_to_bf16_bits((rng.standard_normal(s) * sd).astype(np.float32))
    q, kp, vp = f(Tq, Hq, D), f(Hkv, P, D, sd=D ** -0.5), f(Hkv, P, D, sd=D ** -0.5)
    kn, vn = f(Hkv, Tq, D, sd=D ** -0.5), f(Hkv, Tq, D, sd=D ** -0.5)
    for ns in (0, 3):
        out, lse = ops.partial_draft_attn(*(to_dev(a, "bf16") for a in (q, kp, vp, kn, vn)), scale=D ** -0.5,
                                          num_splits=ns)
        torch.cuda.synchronize()
        ro, rl = oracle.draft_attn_ref(q, kp, vp, kn, vn, D ** -0.5, "bf16")
        check_attn(out, lse, ro, rl, "bf16", f"splits={ns}")
