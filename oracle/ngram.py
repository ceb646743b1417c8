"""N-gram table of the committed text and top-k 4-gram retrieval, by definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

TokenSwift pages: the tool listing's "How it works" retrieves the top-k
candidate 4-grams, which become draft tokens, and after verification updates
the n-gram table; the summary page's "Approach" retrieves n-grams from the
generated text, and its ablation table compares k = 20 with k = 0; the model
card's CLI example sets ``--ngram_topk 20``.

Readings (the pages name the table, not its keying, scoring or update rule):

* The table holds every 4-gram of the committed text, the tokens at positions
  p-3 .. p for each p >= 3, with its count and the last position p at which
  it ended.
* An update after the text grew from n0 to n1 tokens adds the 4-grams ending
  at positions n0 .. n1-1 (those with p >= 3).
* Retrieval for a first token f: the 4-grams whose first token is f, ranked by
  count (higher first), then by last position (more recent first), the first
  k of them (fewer if fewer match). Every position ends one 4-gram, so last
  positions are distinct and the ranking is a total order.
* f is the candidate for the first draft position (the root of the candidate
  tree); each retrieved 4-gram is one chain of four drafts rooted there.
"""
from __future__ import annotations

import numpy as np


def ngram_update(table, tokens, n0, n1):
    """Adds to `table` (dict 4-gram -> [count, last position]) the 4-grams ending at n0 .. n1-1."""
    tokens = [int(t) for t in tokens]
    for p in range(max(n0, 3), n1):
        g = tuple(tokens[p - 3:p + 1])
        if g in table:
            table[g][0] += 1
            table[g][1] = p
        else:
            table[g] = [1, p]
    return table


def ngram_table(tokens):
    """The table of a whole text."""
    return ngram_update({}, tokens, 0, len(tokens))


def retrieve_ref(table, first, k):
    """(grams [m][4], counts [m], last positions [m]) of the top-k 4-grams starting with `first`."""
    hits = [(c, last, g) for g, (c, last) in table.items() if g[0] == int(first)]
    hits.sort(key=lambda h: (-h[0], -h[1]))
    hits = hits[:k]
    grams = np.array([h[2] for h in hits], np.int64).reshape(-1, 4)
    return grams, np.array([h[0] for h in hits], np.int64), np.array([h[1] for h in hits], np.int64)
