"""GPU: ts_attn_merge_and_importance against ts_attn_merge and
ts_kv_importance_score called separately (each pinned to the oracle in
tests/test_gpu_verify.py and tests/test_gpu_partial.py). The one-launch path
runs the same per-workgroup code as the two kernels, so every output must be
bit-identical; shapes outside it take the two launches and must be too."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say
from long_context_kv_ts_amd import ops

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
def test_bit_identical_to_separate_calls(case):
    c = dict(case)
    odt, chunk = c.pop("odt"), c.pop("chunk")
    say(f"fused merge+importance {case}")
    o_part, l_part, q, k = _inputs(5, **c, empty_splits=True)
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
