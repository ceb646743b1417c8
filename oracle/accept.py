"""Acceptance of the verified drafts and the KV-cache commit, by definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

TokenSwift tool listing, "How it works": after the target model has produced
its tokens for every draft position, a draft is valid when its tokens match
the target's exactly; one of the longest valid drafts is picked at random, and
the KV cache is updated with it.

Readings (the pages give the rule, not the indexing):

* The drafts form a forest given by ``parent[]`` (``parent[t]`` in [-1, t);
  anything else counts as a root, the same rule as the attention mask).
* ``target_tok`` has T+1 entries: ``target_tok[0]`` is the target's token for
  the position right after the committed context, and ``target_tok[t+1]`` its
  token for the position right after draft t (produced by the verify pass at
  row t).
* The draft path root -> t is valid when every node on it carries the token
  the target produced at the position before it: a root must equal
  ``target_tok[0]``, any other node a must equal ``target_tok[parent[a] + 1]``.
* Among the valid paths of greatest length, ordered by their last node's
  index, path number ``rand_u32 % count`` is chosen. The random number is drawn
  by the caller and passed in.
* Result: n = the chosen path's length (0 if no root is valid), the path's
  node indices root first, and the bonus token ``target_tok[t_last + 1]``
  (``target_tok[0]`` when n = 0): the target's own token after the accepted
  drafts.
* Commit: cache rows L .. L+n-1 of every KV head receive the K/V rows of the
  path's nodes from the draft buffers, in path order, bit for bit.
"""
from __future__ import annotations

import numpy as np


def _root_path(parent, t):
    """Node indices from the root down to t."""
    path = []
    a = t
    while a >= 0:
        path.append(a)
        p = int(parent[a])
        a = p if -1 <= p < a else -1
    return path[::-1]


def accept_ref(parent, draft_tok, target_tok, rand_u32):
    """(n, path, bonus): brute force over every root-to-node path."""
    parent = np.asarray(parent, dtype=np.int64)
    draft_tok = np.asarray(draft_tok, dtype=np.int64)
    target_tok = np.asarray(target_tok, dtype=np.int64)
    T = len(parent)
    assert len(draft_tok) == T and len(target_tok) == T + 1
    best, cands = 0, []
    for t in range(T):
        path = _root_path(parent, t)
        ok = all(draft_tok[a] == target_tok[(path[i - 1] + 1) if i > 0 else 0]
                 for i, a in enumerate(path))
        if not ok:
            continue
        if len(path) > best:
            best, cands = len(path), [t]
        elif len(path) == best:
            cands.append(t)
    if not cands:
        return 0, [], int(target_tok[0])
    last = cands[int(rand_u32) % len(cands)]
    path = _root_path(parent, last)
    return len(path), path, int(target_tok[last + 1])


def commit_ref(k_cache, v_cache, L, k_draft, v_draft, path):
    """New K/V caches with rows L .. L+n-1 replaced by the path's draft rows."""
    k_new, v_new = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    for i, a in enumerate(path):
        k_new[:, L + i] = k_draft[:, a]
        v_new[:, L + i] = v_draft[:, a]
    return k_new, v_new
