"""GPU: every binding rejects a caller-supplied output or workspace of the wrong
shape, dtype or size with a Python exception before the library is called
(the C ABI sees only addresses, so such a buffer would be written out of
bounds). Nothing here launches a kernel on a bad buffer."""
import pytest
import torch

from gpu_util import DEV, say
from long_context_kv_ts_amd import ops

pytestmark = pytest.mark.gpu


def _bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16, device=DEV)


def _f(*shape):
    return torch.zeros(shape, dtype=torch.float32, device=DEV)


def _i(*shape):
    return torch.zeros(shape, dtype=torch.int32, device=DEV)


def test_verify_outputs_checked():
    say("[binding] verify outputs")
    T, Hq, Hkv, D, L = 8, 8, 2, 128, 256
    q, kc, vc, kd, vd = _bf(T, Hq, D), _bf(Hkv, L, D), _bf(Hkv, L, D), _bf(Hkv, T, D), _bf(Hkv, T, D)
    par = torch.arange(-1, T - 1, dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError, match="out"):
        ops.tree_verify_attn(q, kc, vc, kd, vd, par, out=_bf(T - 1, Hq, D))
    with pytest.raises(TypeError, match="out"):
        ops.tree_verify_attn(q, kc, vc, kd, vd, par, out=_f(T, Hq, D))
    with pytest.raises(ValueError, match="lse"):
        ops.tree_verify_attn(q, kc, vc, kd, vd, par, lse=_f(T))
    with pytest.raises(ValueError, match="workspace"):
        ops.tree_verify_attn(q, kc, vc, kd, vd, par, workspace=torch.empty(256, dtype=torch.uint8, device=DEV))
    S = ops.num_splits(T, Hq, Hkv, D, L, torch.bfloat16)
    with pytest.raises(ValueError, match="o_part"):
        ops.tree_verify_attn_partials(q, kc, vc, kd, vd, par, o_part=_f(S - 1, T, Hq, D))
    with pytest.raises(ValueError, match="l_part"):
        ops.tree_verify_attn_partials(q, kc, vc, kd, vd, par, l_part=_f(S, T, Hq + 1))
    o, l = ops.tree_verify_attn_partials(q, kc, vc, kd, vd, par)
    with pytest.raises(ValueError, match="out"):
        ops.attn_merge(o, l, out=_bf(T, Hq, D // 2))
    with pytest.raises(ValueError, match="lse"):
        ops.attn_merge(o, l, lse=_f(T, Hq, 1))
    torch.cuda.synchronize()


def test_partial_step_outputs_checked():
    say("[binding] partial-KV outputs")
    R, Hq, Hkv, D, L, chunk, k = 4, 32, 8, 128, 64 * 16, 64, 4
    q, kc, vc = _bf(R, Hq, D), _bf(Hkv, L, D), _bf(Hkv, L, D)
    with pytest.raises(ValueError, match="scores"):
        ops.kv_importance_score(q, kc, chunk, scores=_f(Hkv, L // chunk - 1))
    scores = ops.kv_importance_score(q, kc, chunk)
    with pytest.raises(ValueError, match="chunk_idx"):
        ops.kv_topk_select(scores, k, chunk_idx=_i(Hkv, k - 1))
    with pytest.raises(TypeError, match="chunk_score"):
        ops.kv_topk_select(scores, k, chunk_score=_i(Hkv, k))
    idx, _ = ops.kv_topk_select(scores, k)
    with pytest.raises(ValueError, match="k_part"):
        ops.kv_gather(kc, vc, idx, chunk, k_part=_bf(Hkv, k * chunk - 1, D))
    with pytest.raises(TypeError, match="v_part"):
        ops.kv_gather(kc, vc, idx, chunk, v_part=_f(Hkv, k * chunk, D))
    kp, vp = ops.kv_gather(kc, vc, idx, chunk)
    kn, vn = _bf(Hkv, R, D), _bf(Hkv, R, D)
    with pytest.raises(ValueError, match="out"):
        ops.partial_draft_attn(q, kp, vp, kn, vn, out=_bf(R, Hq, D)[:, ::2])
    with pytest.raises(ValueError, match="workspace"):
        ops.partial_draft_attn(q, kp, vp, kn, vn, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError, match="lse"):
        ops.attn_merge_and_importance(_f(4, 8, Hq, D), _f(4, 8, Hq), q, kc, chunk, lse=_f(8))
    torch.cuda.synchronize()


def test_decode_step_outputs_checked():
    say("[binding] decode-step outputs")
    logits = torch.randn((4, 5000), device=DEV)
    with pytest.raises(ValueError, match="parent"):
        ops.build_draft_tree(logits, [1, 3, 3, 3], parent=_i(39))
    with pytest.raises(ValueError, match="workspace"):
        ops.build_draft_tree(logits, [1, 3, 3, 3], workspace=torch.empty(8, dtype=torch.uint8, device=DEV))
    parent, tok, _ = ops.build_draft_tree(logits, [1, 3, 3, 3])
    T = parent.shape[0]
    tl = torch.randn((T + 1, 5000), device=DEV)
    with pytest.raises(ValueError, match="tok"):
        ops.sample_tokens(tl, parent=parent, draft_tok=tok, temperature=0.0, tok=_i(T))
    tgt = ops.sample_tokens(tl, parent=parent, draft_tok=tok, temperature=0.0)
    kc, vc = _bf(2, 50 + T, 128), _bf(2, 50 + T, 128)
    kd, vd = _bf(2, T, 128), _bf(2, T, 128)
    with pytest.raises(ValueError, match="path"):
        ops.accept_commit(parent, tok, tgt, 1, kc, vc, 50, kd, vd, path=_i(T + 1))
    table = ops.NgramTable(DEV, capacity_log2=10, max_entries=512)
    with pytest.raises(ValueError, match="out_tok"):
        table.retrieve(tok[:1], 20, out_tok=_i(20, 3))
    torch.cuda.synchronize()
