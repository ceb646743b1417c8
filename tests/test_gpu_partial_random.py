"""GPU parity of the partial-KV step over a seeded random sweep of shapes:
chunk importance, top-k, gather and the draft attention against the CPU
oracle, and the gather + draft attention launch (ts_kv_gather_and_draft_attn)
bit-identical to the two separate calls. Chunk sizes, grouped heads, recent
queries, head_dim, chunk counts and budgets vary together, so the
combinations the named cases do not pin still meet the contract."""
import numpy as np
import pytest
import torch

from long_context_kv_ts_amd import inputs, ops
import oracle
from gpu_util import check_attn, say, to_dev
from test_gpu_partial import SCORE_REL, topk_matches_with_near_tie_rule

pytestmark = pytest.mark.gpu


def _case(i):
    rng = np.random.default_rng(3000 + i)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
    R = int(rng.integers(1, min(4, 64 // G) + 1))
    chunk = int(rng.choice([16, 32, 64, 64, 100, 128, 256]))
    n_chunks = int(rng.integers(1, 300))
    k = int(rng.integers(1, n_chunks + 1))
    return dict(D=D, Hkv=Hkv, Hq=Hkv * G, R=R, chunk=chunk, L=chunk * n_chunks, k=k,
                n_boost=min(4, k, n_chunks), seed=4000 + i)


CASES = [_case(i) for i in range(20)]


@pytest.mark.parametrize("case", CASES, ids=[f"G{c['Hq'] // c['Hkv']}-Hkv{c['Hkv']}-R{c['R']}-D{c['D']}-chunk{c['chunk']}-"
                                              f"L{c['L']}-k{c['k']}" for c in CASES])
def test_random_partial_steps(case):
    say(f"[random partial] {case}")
    p = inputs.make_partial("random", Hq=case["Hq"], Hkv=case["Hkv"], D=case["D"], L=case["L"], R=case["R"],
                            chunk=case["chunk"], k=case["k"], n_boost=case["n_boost"], seed=case["seed"])
    q, kc, vc = to_dev(p.q, "bf16"), to_dev(p.k_cache, "bf16"), to_dev(p.v_cache, "bf16")
    kn, vn = to_dev(p.k_new, "bf16"), to_dev(p.v_new, "bf16")
    scores = ops.kv_importance_score(q, kc, p.chunk, scale=p.scale)
    idx, val = ops.kv_topk_select(scores, p.k)
    kp, vp = ops.kv_gather(kc, vc, idx, p.chunk)
    out, lse = ops.partial_draft_attn(q, kp, vp, kn, vn, scale=p.scale)
    kp2, vp2, out2, lse2 = ops.kv_gather_and_draft_attn(kc, vc, idx, p.chunk, q, kn, vn, scale=p.scale)
    torch.cuda.synchronize()

    ref_s = oracle.importance_ref(p.q, p.k_cache, p.scale, p.chunk, "bf16")
    gs = scores.cpu().numpy().astype(np.float64)
    assert np.abs(gs - ref_s).max() <= SCORE_REL * np.abs(ref_s).max()

    gidx = idx.cpu().numpy()
    same_prec_idx, same_prec_val = oracle.topk_ref(gs, p.k)
    np.testing.assert_array_equal(gidx, same_prec_idx)
    np.testing.assert_array_equal(val.cpu().numpy(), same_prec_val.astype(np.float32))
    topk_matches_with_near_tie_rule(gidx, ref_s, p.k)

    rkp, rvp = oracle.gather_ref(p.k_cache, p.v_cache, gidx, p.chunk)
    np.testing.assert_array_equal(kp.view(torch.int16).cpu().numpy().view(np.uint16), rkp)
    np.testing.assert_array_equal(vp.view(torch.int16).cpu().numpy().view(np.uint16), rvp)
    ro, rl = oracle.draft_attn_ref(p.q, rkp, rvp, p.k_new, p.v_new, p.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "draft attention")

    # the combined launch: bit-identical to the two calls
    assert torch.equal(kp2.view(torch.int16), kp.view(torch.int16))
    assert torch.equal(vp2.view(torch.int16), vp.view(torch.int16))
    assert torch.equal(out2.view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse2, lse)
