"""Pins for the candidate-tree oracle (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import build_tree_ref
from oracle.tree import topk_tokens

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_example.json")


def test_hand_worked_example():
    ex = json.load(open(GOLDEN))
    parent, tok, cand = build_tree_ref(ex["logits"], ex["shape"])
    assert parent.tolist() == ex["parent"] and tok.tolist() == ex["draft_tok"]
    assert [c.tolist() for c in cand] == ex["cand"]


@pytest.mark.parametrize("shape,nodes", [([1, 3, 3, 3], 40), ([3, 3, 3, 3], 120), ([1, 9, 9, 9], 820)])
def test_node_counts_of_the_pages_tree_shapes(shape, nodes):
    """The ablation table's shapes: 1+3+9+27, 3+9+27+81 and 1+9+81+729 nodes."""
    logits = np.random.default_rng(0).standard_normal((4, 50))
    parent, tok, _ = build_tree_ref(logits, shape)
    assert len(parent) == nodes and (parent < np.arange(nodes)).all()
    assert (parent < 0).sum() == shape[0]


def test_topk_tokens_against_a_full_sort_with_ties():
    rng = np.random.default_rng(1)
    for _ in range(50):
        v = np.round(rng.standard_normal(40), 1)             # many exact ties
        k = int(rng.integers(1, 12))
        ranked = sorted(range(40), key=lambda i: (-v[i], i))
        assert topk_tokens(v, k).tolist() == ranked[:k]


@pytest.mark.parametrize("shape", [[1, 3, 3, 3], [3, 3, 3, 3], [2, 1, 4], [5]])
def test_every_rank_tuple_appears_once_along_root_paths(shape):
    """Walking node t to its root reads the candidates of its rank tuple, and
    every tuple of ranks (one per depth) labels exactly one node."""
    rng = np.random.default_rng(2)
    V = 30
    logits = rng.permutation(len(shape) * V).reshape(len(shape), V).astype(float)   # distinct values
    parent, tok, cand = build_tree_ref(logits, shape)
    seen = set()
    for t in range(len(parent)):
        path = []
        a = t
        while a >= 0:
            path.append(a)
            a = int(parent[a])
        path = path[::-1]
        ranks = tuple(int(np.where(cand[d] == tok[a])[0][0]) for d, a in enumerate(path))
        assert ranks not in seen
        seen.add(ranks)
    expect = sum(int(np.prod(shape[:d + 1])) for d in range(len(shape)))
    assert len(seen) == expect
    depth = [0 if parent[t] < 0 else None for t in range(len(parent))]
    for t in range(len(parent)):
        if parent[t] >= 0:
            depth[t] = depth[parent[t]] + 1
    assert depth == sorted(depth)                                # breadth-first numbering
