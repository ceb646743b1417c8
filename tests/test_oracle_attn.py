"""Pins for the attention oracle (CPU only).

Each test ties ``oracle.verify_attn_ref`` / ``draft_attn_ref`` to something
other than itself: 50-digit brute force with an independently built visibility
set, torch's scaled-dot-product attention (decode and causal forms), closed
forms of softmax, and structural counts of the page's [1,3,3,3] tree.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from long_context_kv_ts_amd import inputs
from oracle import ancestor_mask, draft_attn_ref, verify_attn_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def _rand_case(rng, T, Hq, Hkv, D, L, dtype="f32", parent=None, std=1.0):
    def draw(*shape):
        x = (rng.standard_normal(shape) * std).astype(np.float32)
        return inputs.f32_to_bf16_bits(x) if dtype == "bf16" else x
    if parent is None:
        parent = np.array([-1 if t == 0 or rng.random() < 0.3 else int(rng.integers(0, t))
                           for t in range(T)], dtype=np.int32)
    return dict(q=draw(T, Hq, D), k_cache=draw(Hkv, L, D), v_cache=draw(Hkv, L, D),
                k_draft=draw(Hkv, T, D), v_draft=draw(Hkv, T, D), parent=parent)


def _f64(a):
    if a.dtype == np.uint16:
        return inputs.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# brute force: visibility from root->node paths (children lists + DFS), sums in
# 50-digit arithmetic
# ---------------------------------------------------------------------------
def _paths(parent):
    children = {}
    for t, p in enumerate(parent):
        children.setdefault(int(p), []).append(t)
    paths, stack = {}, [(r, (r,)) for r in children.get(-1, [])]
    while stack:
        node, path = stack.pop()
        paths[node] = path
        stack.extend((c, path + (c,)) for c in children.get(node, []))
    return paths


def _brute(c, scale):
    mpmath.mp.dps = 50
    q, kc, vc, kd, vd = (_f64(c[n]) for n in ("q", "k_cache", "v_cache", "k_draft", "v_draft"))
    T, Hq, D = q.shape
    Hkv, L, _ = kc.shape
    G = Hq // Hkv
    paths = _paths(c["parent"])
    out = np.zeros((T, Hq, D))
    lse = np.zeros((T, Hq))
    for t in range(T):
        for h in range(Hq):
            g = h // G
            keys = [(kc[g, j], vc[g, j]) for j in range(L)] + [(kd[g, a], vd[g, a]) for a in paths[t]]
            s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(x)) * mpmath.mpf(float(y))
                                                  for x, y in zip(q[t, h], k)) for k, _ in keys]
            m = max(s)
            w = [mpmath.exp(x - m) for x in s]
            z = mpmath.fsum(w)
            for d in range(D):
                out[t, h, d] = float(mpmath.fsum(wi * mpmath.mpf(float(v[d])) for wi, (_, v) in zip(w, keys)) / z)
            lse[t, h] = float(m + mpmath.log(z))
    return out, lse


@pytest.mark.parametrize("seed,T,Hq,Hkv,D,L,dtype", [
    (0, 5, 2, 1, 4, 6, "f32"),
    (1, 6, 4, 2, 8, 3, "f32"),
    (2, 4, 2, 2, 8, 8, "bf16"),
    (3, 3, 3, 1, 5, 0, "f32"),     # empty cache: drafts only
])
def test_brute_force_tiny(seed, T, Hq, Hkv, D, L, dtype):
    rng = np.random.default_rng(seed)
    c = _rand_case(rng, T, Hq, Hkv, D, L, dtype)
    scale = 1.0 / math.sqrt(D)
    out, lse = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                               c["parent"], scale, dtype)
    bout, blse = _brute(c, scale)
    np.testing.assert_allclose(out, bout, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, blse, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# reductions to torch's scaled-dot-product attention (CPU, float64)
# ---------------------------------------------------------------------------
def _sdpa(q, k, v, mask, scale, G):
    """q [T][Hq][D], k/v [Hkv][N][D], mask bool [T][N] -> out [T][Hq][D]."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                 # [1][Hq][T][D]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)[None]      # [1][Hq][N][D]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask)[None, None], scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_root_only_is_decode_attention():
    rng = np.random.default_rng(10)
    c = _rand_case(rng, 1, 8, 2, 16, 37, parent=np.array([-1], np.int32))
    out, _ = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                             c["parent"], 0.25, "f32")
    k = np.concatenate([_f64(c["k_cache"]), _f64(c["k_draft"])], axis=1)
    v = np.concatenate([_f64(c["v_cache"]), _f64(c["v_draft"])], axis=1)
    ref = _sdpa(_f64(c["q"]), k, v, np.ones((1, 38), bool), 0.25, 4)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_chain_is_causal_attention_after_prefix():
    rng = np.random.default_rng(11)
    T, L = 7, 29
    c = _rand_case(rng, T, 6, 3, 8, L, parent=np.arange(-1, T - 1, dtype=np.int32))
    out, _ = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                             c["parent"], 0.3, "f32")
    k = np.concatenate([_f64(c["k_cache"]), _f64(c["k_draft"])], axis=1)
    v = np.concatenate([_f64(c["v_cache"]), _f64(c["v_draft"])], axis=1)
    mask = np.concatenate([np.ones((T, L), bool), np.tril(np.ones((T, T), bool))], axis=1)
    ref = _sdpa(_f64(c["q"]), k, v, mask, 0.3, 2)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    # the draft-attention entry is exactly this chain case
    dout, _ = draft_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"], 0.3, "f32")
    np.testing.assert_array_equal(dout, out)


def test_tree_node_equals_causal_attention_along_its_path():
    """Every node of a shuffled [1,3,3,3] tree sees exactly what the last token
    of a causal sequence (cache, then its root-to-node path) sees."""
    rng = np.random.default_rng(12)
    parent = inputs.tree_parents((1, 3, 3, 3), rng)
    T, L, D = len(parent), 19, 8
    c = _rand_case(rng, T, 2, 1, D, L, parent=parent)
    out, _ = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                             parent, 0.35, "f32")
    paths = _paths(parent)
    for t in range(T):
        path = list(paths[t])
        n = len(path)
        k = np.concatenate([_f64(c["k_cache"]), _f64(c["k_draft"])[:, path]], axis=1)
        v = np.concatenate([_f64(c["v_cache"]), _f64(c["v_draft"])[:, path]], axis=1)
        mask = np.concatenate([np.ones((n, L), bool), np.tril(np.ones((n, n), bool))], axis=1)
        ref = _sdpa(_f64(c["q"])[path], k, v, mask, 0.35, 2)
        np.testing.assert_allclose(out[t], ref[-1], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(13)
    parent = inputs.tree_plus_chains_parents(rng)
    T, L, D, Hq, Hkv = len(parent), 50, 8, 4, 2
    c = _rand_case(rng, T, Hq, Hkv, D, L, parent=parent)
    k0 = rng.standard_normal(D).astype(np.float32)
    c["k_cache"][:] = k0
    c["k_draft"][:] = k0
    out, lse = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                               parent, 0.2, "f32")
    paths = _paths(parent)
    vc, vd, q = _f64(c["v_cache"]), _f64(c["v_draft"]), _f64(c["q"])
    for t in range(T):
        n = L + len(paths[t])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            mean_v = (vc[g].sum(0) + vd[g, list(paths[t])].sum(0)) / n
            s0 = 0.2 * float(np.dot(q[t, h], k0.astype(np.float64)))
            np.testing.assert_allclose(out[t, h], mean_v, rtol=1e-12, atol=1e-14)
            assert abs(lse[t, h] - (s0 + math.log(n))) < 1e-12


def test_zero_query_is_uniform():
    rng = np.random.default_rng(14)
    parent = inputs.tree_parents((1, 3, 3, 3), rng)
    c = _rand_case(rng, len(parent), 2, 1, 4, 10, parent=parent)
    c["q"][:] = 0
    _, lse = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                             parent, 0.5, "f32")
    depth = np.array([len(p) for _, p in sorted(_paths(parent).items())])
    np.testing.assert_allclose(lse, np.log(10 + depth)[:, None].repeat(2, 1), rtol=0, atol=1e-14)


def test_one_dominant_key():
    """All keys zero except cached key j*: s* = scale*q.k*, s0 = 0 elsewhere."""
    rng = np.random.default_rng(15)
    T, L, D = 1, 12, 8
    c = _rand_case(rng, T, 1, 1, D, L, parent=np.array([-1], np.int32))
    c["k_cache"][:] = 0
    c["k_draft"][:] = 0
    kstar = rng.standard_normal(D).astype(np.float32) * 3
    c["k_cache"][0, 5] = kstar
    out, lse = verify_attn_ref(c["q"], c["k_cache"], c["v_cache"], c["k_draft"], c["v_draft"],
                               c["parent"], 1.0, "f32")
    s = float(np.dot(_f64(c["q"])[0, 0], kstar.astype(np.float64)))
    n = L + 1
    v = np.concatenate([_f64(c["v_cache"])[0], _f64(c["v_draft"])[0]], axis=0)
    expect = (math.exp(s) * v[5] + (v.sum(0) - v[5])) / (math.exp(s) + n - 1)
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-12, atol=1e-14)
    assert abs(lse[0, 0] - math.log(math.exp(s) + n - 1)) < 1e-12


# ---------------------------------------------------------------------------
# the mask against the page's tree shapes
# ---------------------------------------------------------------------------
def test_tree_shapes_and_visible_counts_match_pages():
    gold = json.load(open(GOLDEN))
    rng = np.random.default_rng(16)
    for entry in gold["tree_shapes"]:
        parent = inputs.tree_parents(entry["shape"], rng)
        assert len(parent) == entry["nodes_derived"]
        assert all(parent[t] < t for t in range(len(parent)))
        vis = ancestor_mask(parent)
        # a node's visible drafts = its depth + 1; levels in order
        counts = vis.sum(1)
        sizes = entry["level_sizes_derived"]
        expect = np.concatenate([np.full(n, d + 1) for d, n in enumerate(sizes)])
        np.testing.assert_array_equal(counts, expect)
        # every non-leaf node has exactly shape[d+1] children
        kids = np.bincount(parent[parent >= 0], minlength=len(parent))
        start = 0
        for d, n in enumerate(sizes[:-1]):
            assert (kids[start:start + n] == entry["shape"][d + 1]).all()
            start += n
    full = inputs.tree_plus_chains_parents(np.random.default_rng(0))
    assert len(full) == gold["draft_rows_derived"]["value"] == 40 + gold["ngram_topk"]["value"] * gold["gamma"]["value"]
    vis = ancestor_mask(full)
    assert vis[:40, :40].sum() == gold["visible_draft_pairs_derived"]["tree_1333"]
    assert vis[40:, 40:].sum() == gold["visible_draft_pairs_derived"]["chains_20x4"]
    assert not vis[40:, :40].any() and not vis[:40, 40:].any()


def test_ancestor_mask_rejects_bad_parents():
    with pytest.raises(ValueError):
        ancestor_mask(np.array([-1, 2, 0], np.int32))
    with pytest.raises(ValueError):
        ancestor_mask(np.array([0], np.int32))
