"""Pins for the n-gram oracle (oracle/ngram.py): a hand-worked example, numpy's
unique-rows count of the sliding windows, incremental updates against the
whole text, and the ranking's total order."""
import json
import os

import numpy as np
import pytest
from numpy.lib.stride_tricks import sliding_window_view

from oracle.ngram import ngram_table, ngram_update, retrieve_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_example.json")


def test_hand_worked_example():
    ex = json.load(open(GOLDEN))
    table = ngram_table(ex["tokens"])
    assert len(table) == ex["distinct"]
    for q in ex["queries"]:
        grams, counts, last = retrieve_ref(table, q["first"], q["k"])
        assert grams.tolist() == q["grams"] and counts.tolist() == q["counts"] and last.tolist() == q["last"], q


@pytest.mark.parametrize("V,n", [(3, 50), (50, 2000), (5000, 20000)])
def test_counts_match_numpy_unique_rows(V, n):
    rng = np.random.default_rng(V)
    tokens = rng.integers(0, V, n)
    table = ngram_table(tokens)
    rows, counts = np.unique(sliding_window_view(tokens, 4), axis=0, return_counts=True)
    assert len(table) == len(rows)
    for r, c in zip(rows, counts):
        assert table[tuple(int(x) for x in r)][0] == c
    assert sum(c for c, _ in table.values()) == n - 3


def test_last_positions_by_brute_force():
    rng = np.random.default_rng(4)
    tokens = rng.integers(0, 4, 300)
    win = sliding_window_view(tokens, 4)
    for g, (_, last) in ngram_table(tokens).items():
        ends = np.nonzero((win == np.array(g)).all(axis=1))[0] + 3
        assert last == ends.max()


def test_incremental_updates_equal_the_whole_text():
    rng = np.random.default_rng(5)
    tokens = rng.integers(0, 6, 500)
    table, n0 = {}, 0
    for n1 in (1, 2, 3, 4, 5, 9, 100, 101, 357, 500):       # growth steps as after each verification
        ngram_update(table, tokens, n0, n1)
        n0 = n1
        assert table == ngram_table(tokens[:n1])


def test_retrieval_is_sorted_filtered_and_truncated():
    rng = np.random.default_rng(6)
    tokens = rng.integers(0, 5, 3000)
    table = ngram_table(tokens)
    for f in range(5):
        grams, counts, last = retrieve_ref(table, f, 20)
        assert len(grams) == min(20, sum(1 for g in table if g[0] == f))
        assert (grams[:, 0] == f).all()
        keys = list(zip(counts.tolist(), last.tolist()))
        assert keys == sorted(keys, reverse=True) and len(set(last.tolist())) == len(last)
        # nothing left out ranks above the last one returned
        worst = keys[-1]
        assert all((c, l) < worst for g, (c, l) in table.items() if g[0] == f and g not in set(map(tuple, grams.tolist())))
    assert retrieve_ref(table, 99, 20)[0].shape == (0, 4)
