"""Candidate tree of draft tokens from the per-position logits, by definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

TokenSwift tool listing, "How it works": one forward pass (the target model
plus its extra linear heads) yields logits for the next 4 positions, and the
candidate drafts are organised as a tree; the summary page's ablation table
compares the tree shapes [1,3,3,3], [3,3,3,3] and [1,9,9,9].

Readings (the pages name the shapes, not the construction):

* shape [k0, k1, k2, k3]: the candidates at depth d are the k_d highest logits
  of position d, ranked by logit, equal logits by lower token id;
* the tree is the Cartesian product of the depths: every node at depth d has
  k_{d+1} children, one per candidate of depth d+1 -- [1,3,3,3] has
  1+3+9+27 = 40 nodes, [3,3,3,3] 120, [1,9,9,9] 820;
* nodes are numbered breadth-first, and inside one depth in lexicographic
  order of the candidate ranks along the root path (so parent[t] < t);
* draft_tok[t] is the token of node t's own depth and rank.
"""
from __future__ import annotations

import itertools

import numpy as np


def topk_tokens(logits_row, k):
    """Token ids of the k highest logits, ties toward the lower id."""
    v = np.asarray(logits_row, dtype=np.float64)
    order = np.lexsort((np.arange(len(v)), -v))      # by -logit, then by id
    return order[:k].astype(np.int64)


def build_tree_ref(logits, shape):
    """(parent [T], draft_tok [T], cand [depth][k]) for tree `shape` over logits [P][V]."""
    logits = np.asarray(logits, dtype=np.float64)
    assert len(shape) <= logits.shape[0]
    cand = [topk_tokens(logits[d], k) for d, k in enumerate(shape)]
    parent, tok, index = [], [], {}
    for d in range(len(shape)):
        for ranks in itertools.product(*[range(k) for k in shape[:d + 1]]):
            index[ranks] = len(parent)
            parent.append(index[ranks[:-1]] if d > 0 else -1)
            tok.append(int(cand[d][ranks[-1]]))
    return np.array(parent, np.int64), np.array(tok, np.int64), cand
