"""GPU parity of ts_build_draft_tree (candidate tree from per-position logits)
against the oracle: bit-exact parent[], draft tokens and ranked candidates."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import DEV as DEV_T, say, to_dev
from long_context_kv_ts_amd import inputs, ops
from oracle import build_tree_ref, widen

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_example.json")
VOCAB = 128256            # LLaMA3.1 vocabulary


def check(logits_host, shape, dtype, label):
    lg = to_dev(logits_host, dtype)
    parent, tok, cand = ops.build_draft_tree(lg, shape)
    torch.cuda.synchronize()
    ref_logits = widen(logits_host, dtype)
    rp, rt, rc = build_tree_ref(ref_logits, shape)
    gp, gt, gc = parent.cpu().numpy(), tok.cpu().numpy(), cand.cpu().numpy()
    say(f"  {label}: T={len(rp)} cand[0]={gc[0, :shape[0]].tolist()}")
    assert np.array_equal(gp, rp), f"{label}: parent"
    assert np.array_equal(gt, rt), f"{label}: draft tokens"
    for d, k in enumerate(shape):
        assert gc[d, :k].tolist() == rc[d].tolist() and (gc[d, k:] == -1).all(), f"{label}: cand[{d}]"
    return parent, tok


def test_hand_worked_example():
    ex = json.load(open(GOLDEN))
    check(np.array(ex["logits"], np.float32), ex["shape"], "f32", "golden")


@pytest.mark.parametrize("shape", [[1, 3, 3, 3], [3, 3, 3, 3], [1, 9, 9, 9]])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pages_shapes_full_vocabulary(shape, dtype):
    """The ablation table's tree shapes over a 128,256-token vocabulary; bf16
    logits carry many exact ties."""
    rng = np.random.default_rng(len(shape) * 10 + shape[1])
    logits = (rng.standard_normal((4, VOCAB)) * 3).astype(np.float32)
    if dtype == "bf16":
        logits = inputs.f32_to_bf16_bits(logits)
    check(logits, shape, dtype, f"{shape} {dtype}")


def test_ties_and_small_vocabularies():
    rng = np.random.default_rng(7)
    for V in (1, 3, 16, 17, 1000, 1025):
        P = 5
        logits = np.round(rng.standard_normal((P, V)), 0).astype(np.float32)   # heavy ties
        logits[:, ::7] = -0.0
        shape = [int(min(V, k)) for k in rng.integers(1, 17, P)]
        while sum(int(np.prod(shape[:d + 1])) for d in range(len(shape))) > 1024:
            shape = shape[:-1]
        check(logits, shape, "f32", f"V={V} shape={shape}")


def test_tree_feeds_verify():
    """The [1,3,3,3] tree built on the GPU is a valid parent[] for the verify
    call: its attention matches the oracle's on that forest."""
    from gpu_util import check_attn
    from oracle import verify_attn_ref
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((4, 5000)).astype(np.float32)
    parent, _ = check(logits, [1, 3, 3, 3], "f32", "tree for verify")
    c = inputs.make_verify("tree", dtype="bf16", Hq=8, Hkv=2, D=128, L=700, seed=11, with_chains=False)
    par = parent.cpu().numpy().astype(np.int32)
    assert len(par) == c.T
    out, lse = ops.tree_verify_attn(to_dev(c.q, "bf16"), to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16"),
                                    to_dev(c.k_draft, "bf16"), to_dev(c.v_draft, "bf16"), parent, scale=c.scale)
    torch.cuda.synchronize()
    ro, rl = verify_attn_ref(c.q, c.k_cache, c.v_cache, c.k_draft, c.v_draft, par, c.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "verify on the built tree")


def test_many_slices_and_reused_workspace():
    """Vocabularies that split into several slices (ragged last slice, odd
    slice starts for bf16, the 64-slice cap above 262,144 tokens), with one
    workspace reused across calls and filled with garbage beforehand."""
    rng = np.random.default_rng(21)
    ws = ops.alloc_workspace(int(ops.lib().ts_build_draft_tree_workspace(300001, 4)), DEV_T)
    ws.fill_(0xFF)
    for V, dtype in ((4097, "f32"), (8195, "bf16"), (128257, "bf16"), (300001, "f32")):
        logits = (rng.standard_normal((4, V)) * 2).astype(np.float32)
        # the best tokens of a row sit at both ends and on slice edges
        logits[:, [0, V - 1, V // 2]] = 50.0
        if dtype == "bf16":
            logits = inputs.f32_to_bf16_bits(logits)
        lg = to_dev(logits, dtype)
        shape = [3, 4, 2, 5]
        parent, tok, cand = ops.build_draft_tree(lg, shape, workspace=ws)
        torch.cuda.synchronize()
        rp, rt, rc = build_tree_ref(widen(logits, dtype), shape)
        say(f"  V={V} {dtype}: cand[0]={cand[0, :3].tolist()}")
        assert np.array_equal(parent.cpu().numpy(), rp) and np.array_equal(tok.cpu().numpy(), rt), f"V={V}"
        for d, k in enumerate(shape):
            assert cand[d, :k].cpu().tolist() == rc[d].tolist(), f"V={V} cand[{d}]"


def test_largest_tree_feeds_verify():
    """[1,9,9,9]: the 820-node tree built on the GPU drives the verify call past
    256 drafts, against the oracle."""
    from gpu_util import check_attn
    from oracle import verify_attn_ref
    rng = np.random.default_rng(19)
    logits = rng.standard_normal((4, 3000)).astype(np.float32)
    parent, _ = check(logits, [1, 9, 9, 9], "f32", "[1,9,9,9] for verify")
    par = parent.cpu().numpy().astype(np.int32)
    assert len(par) == 820
    c = inputs.make_verify("tree1999", dtype="bf16", Hq=8, Hkv=2, D=128, L=600, seed=21, with_chains=False,
                           parent=par)
    out, lse = ops.tree_verify_attn(to_dev(c.q, "bf16"), to_dev(c.k_cache, "bf16"), to_dev(c.v_cache, "bf16"),
                                    to_dev(c.k_draft, "bf16"), to_dev(c.v_draft, "bf16"), parent, scale=c.scale)
    torch.cuda.synchronize()
    ro, rl = verify_attn_ref(c.q, c.k_cache, c.v_cache, c.k_draft, c.v_draft, par, c.scale, "bf16")
    check_attn(out, lse, ro, rl, "bf16", "verify on the built [1,9,9,9] tree")
